// proj.hip - INT4 projection kernels (gfx950): QKV, O, gate/up, down.
//
// y[m][n] = sum_g s[n][g] * sum_{k in g} (u[n][k] - 8) * x[m][k]
// ("how it differs": group scales applied after accumulation).
//
// M = 1: register-streaming GEMV (gemv.h).  Each 64-lane wave streams 1 KiB
//   atoms (16 rows x 128 k, one 16-byte load per lane), decodes the nibbles
//   as exact fp16 subnormals (the B operand of four f16 MFMA 16x16x32, one
//   per 32 k) against range-scaled fp16 x, staged in LDS and broadcast to
//   every row of the A operand, so each lane gets the dot of its atom row.
// M = 2..3 (when x fits the kernel's staging; the kernel takes up to 8):
//   the same stream with rows 0..M-1 of x in rows 0..M-1 of the A operand
//   (gemv_rows.h).
// Otherwise (M <= 32): skinny GEMM on bf16 MFMA 16x16x32, computed as
//   sum_g s[n][g] * (A[n][g] - 136 * X[m][g]) where A accumulates
//   (128 + u) * x from the bf16 magic-exponent decode of each nibble and X
//   is the group sum of x (one more MFMA against ones); the scale and the
//   136 correction are applied once per group after the 128-wide
//   accumulation.  Large-K projections may split K across workgroups
//   through the step workspace (the last slice to arrive reduces).
//
// Both split K across the waves of a workgroup, reduce in LDS and run the
// epilogue once per output from an LDS tile:
//   QKV : rho1 (from the staged input), RoPE on q/k pairs, q fp32, k/v bf16
//   O   : h = x + y (fp32 and bf16 copies)
//   GU  : rho2, a = silu(gate) * up (bf16)
//   DOWN: out = h + y (bf16)
#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "gemv.h"
#include "gemv_rows.h"
#include "i4d_internal.h"
#include "proj.h"

namespace i4d {

constexpr int kMaxLdsBytes = 160 * 1024;

// ---------------------------------------------------------------------------
// M = 1: stand-alone GEMV kernel
// ---------------------------------------------------------------------------

template <int EPI, int NW, int U, int GPW>
__global__ __launch_bounds__(NW * 64) void proj_gemv_kernel(ProjArgs a, GemvPlan pl) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nstrips = a.Np / kStrip;
  const int strip0 = blockIdx.x * pl.SP;
  gemv_body<EPI, NW, U, GPW, false>(a, pl, strip0, min(pl.SP, nstrips - strip0), smem, NoWait());
}

// M = 2..8 rows: the M = 1 stream with x rows in the A operand's rows
template <int EPI, int NW, int U, int GPW, int XMAX>
__global__ __launch_bounds__(NW * 64) void proj_gemv_rows_kernel(ProjArgs a, GemvPlan pl) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nstrips = a.Np / kStrip;
  const int strip0 = blockIdx.x * pl.SP;
  gemv_rows_body<EPI, NW, U, GPW, XMAX>(a, pl, strip0, min(pl.SP, nstrips - strip0), smem);
}

// ---------------------------------------------------------------------------
// M = 2..32: bf16 MFMA skinny GEMM
// ---------------------------------------------------------------------------
//
// A workgroup of 8 waves owns SP strips (16 output rows each) and one of
// KS slices of K; the waves split the slice (wave w takes every 8th group
// from w).  For each of its groups a wave loads the x rows of the group
// (T tiles of 16 rows, one group ahead, row-contiguous), turns them into
// B operands of the MFMA through its own LDS rows, and reuses them for the
// SP atoms of the group, which stream through a ring of D groups of
// outstanding 16-byte loads.  The atom lane layout is the A operand.
// Scales are staged in LDS per workgroup, transposed so a lane reads its 4
// rows of a group at once; the waves' partial tiles are summed in LDS in a
// fixed order.

constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyMaxWorkgroups = 256;
constexpr int kScaleLoads = 4;  // 16-byte scale loads per lane: SP * GPW <= 128

struct SkinnyPlan {
  int SP;   // strips per workgroup
  int KS;   // K slices (workgroups per strip set; > 1 needs the split buffers)
  int GPW;  // groups per wave in the longest slice
  int D;    // groups of atoms in flight per wave
};

// floats per (strip set, slice) in the split buffer: the partial tile
// [SP*16][32] and the slice's sums of squares [32]
__host__ __device__ inline size_t split_block_floats(int SP) { return (size_t)SP * 16 * 32 + 32; }

// x rows staged per wave: 256 bytes of a group plus 16 bytes of padding, so
// that operand reads (16 rows at a 272-byte stride) hit distinct banks
constexpr int kXRow = 272;

// LDS: sums of squares [NW][T*16] f32 | rho [T*16] | tile [SP*16][T*16] |
// then either the waves' scales [NW][SP * GPW + 1][16] fp16 (the last row
// zero) + x staging [NW][16T][kXRow bytes] (main loop) or partial tiles
// [4][SP*16][T*16+4] f32 (reduction)
inline size_t skinny_lds_bytes(int GW, int SP, int T) {
  const size_t loop = (size_t)kSkinnyWaves * (SP * GW + 1) * kStrip * 2 + (size_t)kSkinnyWaves * 16 * T * kXRow;
  const size_t reduce = (size_t)4 * SP * 16 * (T * 16 + 4) * 4;
  return (size_t)kSkinnyWaves * T * 16 * 4 + (size_t)T * 16 * 4 + (size_t)SP * 16 * T * 16 * 4 +
         std::max(loop, reduce);
}

template <int EPI, int SP, int T, int D, bool P>
__global__ __launch_bounds__(kSkinnyWaves * 64) void proj_skinny_kernel(ProjArgs a, SkinnyPlan pl) {
  constexpr int NW = kSkinnyWaves;
  constexpr int U = D * SP;  // D groups of atoms in flight
  extern __shared__ __align__(16) unsigned char smem[];
  const int K = a.K, G = a.G, M = a.M;
  float* sqw = reinterpret_cast<float*>(smem);                                   // [NW][T*16]
  float* rho_s = sqw + NW * T * 16;                                              // [T*16]
  float* ot = rho_s + T * 16;                                                    // [SP*16][M]
  uint16_t* sc = reinterpret_cast<uint16_t*>(ot + SP * 16 * T * 16);             // [NW][SP][GPW][16]
  unsigned char* xst = reinterpret_cast<unsigned char*>(sc + (size_t)NW * (SP * pl.GPW + 1) * kStrip);  // [NW][16T][kXRow]
  float* red = reinterpret_cast<float*>(sc);  // [4][SP*16][T*16+4], over sc and xst once the waves are done

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int nstrips = a.Np / kStrip;
  const int KS = pl.KS;
  const int ntiles = (nstrips + SP - 1) / SP * KS;
  // A tile is (strip set, K slice); the slice is groups [gs0, gs0 + Gs).
  // Wave w takes groups w, w + NW, w + 2 NW, ... of the slice (the waves
  // of a workgroup read neighbouring atoms of a strip at the same time);
  // groups past the wave's share (padding to a multiple of D) re-read its
  // last group and are weighted by zero.  P: persistent workgroups take
  // tiles blockIdx.x, + gridDim.x, ...; the last D groups of a tile refill
  // the ring with the next tile's first atoms.
  struct Tile {
    int set, ks, strip0, ns, gs0, Gs, gpw;
  };
  auto tile_of = [&](int t) {
    Tile g;
    g.set = t / KS;
    g.ks = t - g.set * KS;
    g.strip0 = g.set * SP;
    g.ns = min(SP, nstrips - g.strip0);
    g.gs0 = g.ks * G / KS;
    g.Gs = (g.ks + 1) * G / KS - g.gs0;
    g.gpw = max(0, (g.Gs - wave + NW - 1) / NW);
    return g;
  };
  int tile = blockIdx.x;
  Tile cur = tile_of(tile);
  auto group_of_t = [&](const Tile& g, int gi) {
    return g.gs0 + min(wave + NW * min(gi, max(g.gpw - 1, 0)), g.Gs - 1);
  };

  // ring of atoms: slot d * SP + s holds strip s of a group gi with
  // gi % D == d
  auto atom_ptr_t = [&](const Tile& g, int gi, int s) -> const uint8_t* {
    const int t = min(g.strip0 + min(s, g.ns - 1), nstrips - 1);
    return a.codes + ((size_t)t * G + group_of_t(g, gi)) * kAtomBytes + (size_t)lane * 16;
  };
  auto atom_ptr = [&](int gi, int s) { return atom_ptr_t(cur, gi, s); };
  // Each wave stages the scales of its own atoms (SP strips x GW groups,
  // 32 bytes per atom in the [strip][group][row] layout) in its own LDS
  // rows: requested first (they are needed first), no workgroup barrier.
  // Item i of a wave is half i % 2 of atom i / 2; at most kScaleLoads
  // 16-byte loads per lane (items past the wave's atoms re-read valid ones).
  const int GW = pl.GPW;
  auto scale_item = [&](int q, int& s, int& gi, int& half) {
    const int idx = min(lane + q * 64, 2 * SP * GW - 1);
    const int at = idx >> 1;
    half = idx & 1;
    s = at / GW;
    gi = at % GW;
  };
  u32x4_t scv[kScaleLoads];
  auto load_scales = [&](const Tile& g) {
#pragma unroll
    for (int q = 0; q < kScaleLoads; ++q) {
      int s, gi, half;
      scale_item(q, s, gi, half);
      const int t = min(g.strip0 + min(s, g.ns - 1), nstrips - 1);
      scv[q] = load16(a.scales + ((size_t)t * G + group_of_t(g, gi)) * kStrip + 8 * half);
    }
  };
  load_scales(cur);

  // x rows of one group as B operands: lane (col r, quarter j) holds row
  // 16 t + r, k = 128 g + 32 kb + 8 j .. +7.  Columns past M re-read row
  // M - 1 (unconditional loads keep the wait counts exact); their outputs
  // are never stored.
  // Global reads of x are row-contiguous (load q of a wave covers rows
  // 4q .. 4q+3, 256 bytes each: whole cache lines); the wave transposes
  // them through its own LDS rows into the operand layout.
  auto load_xs_t = [&](const Tile& tg, u32x4_t (&xs)[4 * T], int gi) {
    const int g = group_of_t(tg, gi);
#pragma unroll
    for (int q = 0; q < 4 * T; ++q) {
      const int m = min(4 * q + j, M - 1);
      xs[q] = load16(a.x + (size_t)m * K + 128 * g + 8 * r);
    }
  };
  auto load_xs = [&](u32x4_t (&xs)[4 * T], int gi) { load_xs_t(cur, xs, gi); };
  unsigned char* xw = xst + (size_t)wave * (16 * T) * kXRow;
  auto stage_bx = [&](const u32x4_t (&xs)[4 * T], u32x4_t (&bx)[T][4]) {
#pragma unroll
    for (int q = 0; q < 4 * T; ++q) *reinterpret_cast<u32x4_t*>(xw + (4 * q + j) * kXRow + 16 * r) = xs[q];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        bx[t][kb] = *reinterpret_cast<const u32x4_t*>(xw + (16 * t + r) * kXRow + 64 * kb + 16 * j);
  };
  // The first group's x is requested before the first atoms, the order in
  // which the loop requests them (x one group ahead, then the refills):
  // the wait counts the compiler derives at the loop head hold for both
  // ways in, so the head waits for x only and not for the refills issued
  // behind it (with the atoms first, every group began by draining them).
  u32x4_t xs[4 * T];
  load_xs(xs, 0);
  u32x4_t ring[U];
#pragma unroll
  for (int k = 0; k < U; ++k) ring[k] = load16_stream(atom_ptr(k / SP, k % SP));

  constexpr int RS = T * 16 + 4;
  uint16_t* scw = sc + (size_t)wave * (SP * GW + 1) * kStrip;  // this wave's [SP][GW][16] + a zero row
  for (;;) {
  const int set = cur.set, strip0 = cur.strip0, ns = cur.ns, gpw = cur.gpw;
#pragma unroll
  for (int q = 0; q < kScaleLoads; ++q) {
    int s, gi, half;
    scale_item(q, s, gi, half);
    *reinterpret_cast<u32x4_t*>(&scw[(s * GW + gi) * kStrip + 8 * half]) = scv[q];
  }
  if (lane < 2) *reinterpret_cast<u32x4_t*>(&scw[SP * GW * kStrip + 8 * lane]) = u32x4_t{0u, 0u, 0u, 0u};

  const u32x4_t ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const bf16x8_t ones = bitcast<bf16x8_t>(ones_u);
  f32x4_t acc[SP][T];
#pragma unroll
  for (int s = 0; s < SP; ++s)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[s][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float sq[T];
#pragma unroll
  for (int t = 0; t < T; ++t) sq[t] = 0.f;

  // one group: column sums and sums of squares of x, then its SP atoms;
  // each consumed slot is refilled with the same strip D groups ahead
  // refill mode: 0 none, 1 the same strip D groups ahead, 2 the next
  // tile's atom of this slot
  auto do_group = [&](auto refill, const u32x4_t (&bxg)[T][4], const int gi, const int d, const Tile& nx) {
    const bool valid = gi < gpw;
    // X[t] = -136 * (column sums of x): the accumulator start of every atom
    f32x4_t X[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      X[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      float q = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        X[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, bitcast<bf16x8_t>(bxg[t][kb]), X[t], 0, 0, 0);
        if (needs_rho<EPI>())
#pragma unroll
          for (int e = 0; e < 4; ++e)
            q = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(bxg[t][kb][e]), bitcast<bf16x2_t>(bxg[t][kb][e]), q,
                                                false);
      }
      if (needs_rho<EPI>()) sq[t] += valid ? q : 0.f;
      X[t] *= -136.0f;
    }
    // this lane's four scales of atom s (a padding group reads the zero
    // row); at two x tiles all SP pairs are read at the start of the group,
    // so no atom waits on its own LDS read (measured 1.2 us faster at 70B,
    // 32 rows; at one x tile, per atom)
    auto scale_pair = [&](int s) {
      return *reinterpret_cast<const u32x2_t*>(&scw[(valid ? s * GW + min(gi, GW - 1) : SP * GW) * kStrip + 4 * j]);
    };
    u32x2_t svs[T == 2 ? SP : 1];
    if constexpr (T == 2)
#pragma unroll
      for (int s = 0; s < SP; ++s) svs[s] = scale_pair(s);
#pragma unroll
    for (int s = 0; s < SP; ++s) {
      const int k = d * SP + s;
      bf16x8_t A[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) A[kb] = dword_to_bf16x8_biased(ring[k][kb]);
      // refill only after the decode has read the slot, so that the new
      // atom lands in the same registers (no copies or waits on the loop's
      // back edge): the empty asm orders the decode before the load
      asm volatile("" : "+v"(A[0]), "+v"(A[1]), "+v"(A[2]), "+v"(A[3])::"memory");
      if constexpr (decltype(refill)::value == 1) ring[k] = load16_stream(atom_ptr(gi + D, s));
      if constexpr (decltype(refill)::value == 2) ring[k] = load16_stream(atom_ptr_t(nx, d, s));
      const u32x2_t sv = T == 2 ? svs[s] : scale_pair(s);
      float scl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) scl[i] = f16_bits_to_f32((uint16_t)(sv[i >> 1] >> (16 * (i & 1))));
#pragma unroll
      for (int t = 0; t < T; ++t) {
        f32x4_t ag = X[t];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[kb], bitcast<bf16x8_t>(bxg[t][kb]), ag, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[s][t][i] = fmaf(scl[i], ag[i], acc[s][t][i]);
      }
      // one atom's decoded operands live at a time where registers are
      // short (the persistent variants); elsewhere the next atom's decode
      // may overlap this one's MFMAs
      if constexpr (P) __builtin_amdgcn_sched_barrier(0);
    }
    // every read of this group's x is done before the next group's x loads
    // (into the same registers) are issued
#pragma unroll
    for (int s = 0; s < SP; ++s)
#pragma unroll
      for (int t = 0; t < T; ++t) asm volatile("" : "+v"(acc[s][t]));
#pragma unroll
    for (int t = 0; t < T; ++t) asm volatile("" : "+v"(sq[t])::"memory");
  };
  // all but the last D groups refill the ring; the last D consume what is
  // in flight, so no load is still outstanding when the waves meet
  const int ngr = (gpw + D - 1) / D * D;
  int gb = 0;
  u32x4_t bx[T][4];
  for (; gb < ngr - D; gb += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      // the next group's x before this group's refills: the wait for x
      // then leaves the refills (D groups ahead) in flight
      // staging x and requesting the next group's x at raised wave
      // priority: the loads leave before the other waves' atom chains take
      // the issue slots (70B M = 32 step 161.9 -> 159.7 us alternating on
      // one box; no change at 8B M = 32 or 70B M = 16)
      __builtin_amdgcn_s_setprio(2);
      stage_bx(xs, bx);
      __builtin_amdgcn_sched_barrier(0);
      load_xs(xs, gb + d + 1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      do_group(std::integral_constant<int, 1>(), bx, gb + d, d, cur);
      // keep the scheduler from hoisting later groups' loads (register
      // pressure) across the group boundary
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const int nxt_tile = tile + (int)gridDim.x;
  const bool has_next = P && nxt_tile < ntiles;
  const Tile nx = tile_of(has_next ? nxt_tile : tile);
  auto tail = [&](auto mode) {
    constexpr int MODE = decltype(mode)::value;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      stage_bx(xs, bx);
      __builtin_amdgcn_sched_barrier(0);
      if (d + 1 < D) load_xs(xs, gb + d + 1);
      else if (MODE == 2) load_xs_t(nx, xs, 0);
      __builtin_amdgcn_sched_barrier(0);
      do_group(mode, bx, gb + d, d, nx);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (P && has_next) {
    if (ngr > 0) {
      tail(std::integral_constant<int, 2>());
    } else {
      // no groups in this tile for this wave: request the next tile directly
      load_xs_t(nx, xs, 0);
#pragma unroll
      for (int k = 0; k < U; ++k) ring[k] = load16_stream(atom_ptr_t(nx, k / SP, k % SP));
    }
    load_scales(nx);
  } else if (ngr > 0) {
    tail(std::integral_constant<int, 0>());
  }

  // partial tiles: lane holds rows 4j+i of column r of each tile.  Waves
  // 0-3 store theirs, then waves 4-7 add theirs to the same slots (plain
  // LDS reads and writes: LDS float atomics are slow); the row stride RS
  // puts the four row quarters of a store on distinct banks.
  auto slot = [&](int s, int t, int i) { return (((wave & 3) * SP + s) * 16 + 4 * j + i) * RS + t * 16 + r; };
  lds_barrier();  // every wave is past its last read of sc and xst
  if (wave < 4) {
#pragma unroll
    for (int s = 0; s < SP; ++s)
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[slot(s, t, i)] = acc[s][t][i];
  }
  lds_barrier();
  if (wave >= 4) {
#pragma unroll
    for (int s = 0; s < SP; ++s)
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[slot(s, t, i)] += acc[s][t][i];
  }
  if (needs_rho<EPI>()) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float v = sq[t];
      v += lane_xor(v, 16, lane);
      v += lane_xor(v, 32, lane);
      if (j == 0) sqw[wave * T * 16 + t * 16 + r] = v;
    }
  }
  __syncthreads();
  auto red_sum = [&](int row, int m) {
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) v += red[((q * SP) * 16 + row) * RS + m];
    return v;
  };
  auto sq_sum = [&](int m) {
    float v = 0.f;
    for (int w = 0; w < NW; ++w) v += sqw[w * T * 16 + m];
    return v;
  };
  if (KS == 1) {
    for (int idx = tid; idx < ns * 16 * M; idx += NW * 64) ot[idx] = red_sum(idx / M, idx % M);
    if (tid < M) rho_s[tid] = needs_rho<EPI>() ? 1.0f / sqrtf(sq_sum(tid) / (float)K + a.eps) : 1.0f;
  } else {
    // split K: publish this slice's tile and sums of squares (coherent
    // stores), count the slice in; the last slice of the set to arrive sums
    // all KS of them in slice order and runs the epilogue
    const size_t blk = split_block_floats(SP);
    float* part = a.split_part + (size_t)tile * blk;
    const int n4 = ns * 16 * M / 4;  // the tile as 16-byte pieces
    for (int i4 = tid; i4 < n4; i4 += NW * 64) {
      u32x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(red_sum((4 * i4 + e) / M, (4 * i4 + e) % M));
      st_coh16(part, (uint32_t)i4 * 16, (uint32_t)blk * 4, v);
    }
    if (needs_rho<EPI>() && tid < M) st_coh(&part[SP * 16 * 32 + tid], sq_sum(tid));
    wait_vmem();
    __syncthreads();
    int* flag = reinterpret_cast<int*>(rho_s);
    if (tid == 0) {
      const unsigned prev = atomic_add_agent(&a.split_cnt[set], 1u);
      const bool last = prev == (unsigned)(KS - 1);
      if (last) __hip_atomic_store(&a.split_cnt[set], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *flag = last ? 1 : 0;
    }
    __syncthreads();
    if (*flag == 0) {
      if (!has_next) return;
      // the next tile's scale writes come after every wave read the flag
      __syncthreads();
      tile = nxt_tile;
      cur = nx;
      continue;
    }
    __syncthreads();  // every thread has read the flag before rho_s is reused
    // slices summed in order 0 .. KS-1, four loads in flight at a time
    // (slices past KS read slice KS-1 and add zero)
    const float* part0 = a.split_part + (size_t)set * KS * blk;
    const uint32_t set_bytes = (uint32_t)(KS * blk * 4);
    for (int i4 = tid; i4 < n4; i4 += NW * 64) {
      f32x4_t v = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < KS; k0 += 4) {
        u32x4_t p[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          p[q] = ld_coh16(part0, (uint32_t)((min(k0 + q, KS - 1) * blk + 4 * i4) * 4), set_bytes);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t pv = bitcast<f32x4_t>(p[q]);
          if (k0 + q < KS) v += pv;
        }
      }
      *reinterpret_cast<f32x4_t*>(&ot[4 * i4]) = v;
    }
    if (tid < M) {
      float v = 0.f;
      if (needs_rho<EPI>())
        for (int k = 0; k < KS; ++k) v += ld_coh(&part0[(size_t)k * blk + SP * 16 * 32 + tid]);
      rho_s[tid] = needs_rho<EPI>() ? 1.0f / sqrtf(v / (float)K + a.eps) : 1.0f;
    }
  }
  __syncthreads();
  run_epilogue<EPI>(a, strip0, ns, ot, rho_s);
  if (!has_next) return;
  tile = nxt_tile;
  cur = nx;
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------

// M = 2..32 launch shape.  Each workgroup (8 waves) takes SP strips and
// one of KS slices of K.  More strips per workgroup means fewer re-reads of
// x; more slices means more workgroups (and partial tiles to reduce).  The
// plan takes the (SP, KS) that keeps the most CUs busy over the rounds of
// workgroups (ties to more strips), with KS > 1 only when `split_bytes` of
// split buffer are at hand and each wave gets at least one group.  D groups
// of atoms are in flight per wave: one group from four strips up (from two
// at two x tiles), else two groups.  The registers a deeper ring would hold
// go to overlapping consecutive atoms (the decode of the next during the
// MFMAs of this one): alternating on one box, the step at 32 rows took 81
// us against 86 (8B) and 165 against 169 (70B) with the former D = 2 (4 at
// one strip), at 16 rows 121 against 133 (70B) and 67 against 69 (8B) with
// the former D = 2 (4 at two or three strips), and at 8 and 16 rows on the
// 8B shape 1.5 us less with two groups at one strip than with the former
// 4 (8 for the down projection).
static SkinnyPlan skinny_plan(int nstrips, int G, int T, size_t split_bytes) {
  SkinnyPlan best{};
  double best_score = -1.0;
  for (int SP : {7, 5, 4, 3, 2, 1}) {
    const int nsets = (nstrips + SP - 1) / SP;
    int KS = 1;
    if (split_bytes) {
      KS = std::max(1, std::min(256 / nsets, G / kSkinnyWaves));
      while (KS > 1 && (size_t)nsets * KS * split_block_floats(SP) * sizeof(float) > split_bytes) --KS;
    }
    const int gs_max = (G + KS - 1) / KS;
    const int gw = (gs_max + kSkinnyWaves - 1) / kSkinnyWaves;
    if (2 * SP * gw > kScaleLoads * 64 || skinny_lds_bytes(gw, SP, T) > (size_t)kMaxLdsBytes) continue;
    const int W = nsets * KS, rounds = (W + 255) / 256;
    const double score = (double)W / (256.0 * rounds);
    if (score > best_score + 1e-9) {
      best_score = score;
      best.SP = SP;
      best.KS = KS;
      best.GPW = gw;
    }
  }
  best.D = (best.SP >= 4 || (T == 2 && best.SP >= 2)) ? 1 : 2;
  return best;
}

// M = 1 launch shape.  16 waves per workgroup when that leaves at most 4
// groups per wave (x kept in registers), else as few groups per wave as
// the divisors of G allow; strips per workgroup so that about one
// workgroup of 16 waves per CU streams the matrix.
static GemvPlan gemv_plan(int nstrips, int G) {
  GemvPlan p;
  p.NW = 16;
  while (p.NW > 4 && (G % p.NW || G < p.NW)) p.NW /= 2;
  p.GPW = (G + p.NW - 1) / p.NW;
  const int slots = 256 * (16 / p.NW);  // resident workgroups at 16 waves per CU
  p.SP = std::max(1, (nstrips + slots - 1) / slots);
  return p;
}

// The multi-row GEMV keeps 4 atoms per wave in flight at every group count
// (8 at one or two groups per wave and with x from LDS measured slower:
// 8B-shape step at M = 2 49.3 against 45.4 us, alternating on one box).
template <int EPI, int NW>
static void launch_gemv_rows(const ProjArgs& a, const GemvPlan& p, size_t lds, int grid, hipStream_t st) {
  constexpr int X = kRowsXMax;
  switch (gemv_reg_groups(p, a.G)) {
    case 1: hipLaunchKernelGGL((proj_gemv_rows_kernel<EPI, NW, 4, 1, X>), dim3(grid), dim3(NW * 64), lds, st, a, p); break;
    case 2: hipLaunchKernelGGL((proj_gemv_rows_kernel<EPI, NW, 4, 2, X>), dim3(grid), dim3(NW * 64), lds, st, a, p); break;
    case 4: hipLaunchKernelGGL((proj_gemv_rows_kernel<EPI, NW, 4, 4, X>), dim3(grid), dim3(NW * 64), lds, st, a, p); break;
    default:
      hipLaunchKernelGGL((proj_gemv_rows_kernel<EPI, NW, 4, 0, kRowsXMax>), dim3(grid), dim3(NW * 64), lds, st, a, p);
  }
}

template <int EPI, int NW>
static void launch_gemv(const ProjArgs& a, const GemvPlan& p, size_t lds, int grid, hipStream_t st) {
  // x in registers (GPW > 0) needs every wave to own exactly GPW groups
  if (a.G % NW != 0)
    hipLaunchKernelGGL((proj_gemv_kernel<EPI, NW, 8, 0>), dim3(grid), dim3(NW * 64), lds, st, a, p);
  else if (p.GPW == 1)
    hipLaunchKernelGGL((proj_gemv_kernel<EPI, NW, 8, 1>), dim3(grid), dim3(NW * 64), lds, st, a, p);
  else if (p.GPW == 2)
    hipLaunchKernelGGL((proj_gemv_kernel<EPI, NW, 8, 2>), dim3(grid), dim3(NW * 64), lds, st, a, p);
  else if (p.GPW == 4)
    hipLaunchKernelGGL((proj_gemv_kernel<EPI, NW, 4, 4>), dim3(grid), dim3(NW * 64), lds, st, a, p);
  else  // other group counts: x from LDS, 4 atoms in flight (70B down, 224 groups: step 91.8 -> 91.1 us against 8)
    hipLaunchKernelGGL((proj_gemv_kernel<EPI, NW, 4, 0>), dim3(grid), dim3(NW * 64), lds, st, a, p);
}

// split buffer bytes usable by a projection (0: no split of K)
// Splitting K trades x re-reads for a reduction tail (publish, count,
// sum, then the epilogue) of several microseconds; it pays only when each
// unsplit workgroup would read more than kSplitMinXBytes of x.
constexpr size_t kSplitMinXBytes = 512 * 1024;

static size_t split_bytes_of(const ProjArgs& a) {
  if (!a.split_part || !a.split_cnt || (size_t)a.M * a.K * 2 <= kSplitMinXBytes) return 0;
  return a.split_bytes;
}

// The launch shape of one projection: the M = 1 GEMV, the multi-row GEMV
// (rows) or the skinny MFMA kernel, with its plan, LDS bytes and grid.
struct ProjLaunch {
  bool gemv;
  bool rows;  // gemv with 2..8 rows of x
  GemvPlan g;
  SkinnyPlan s;
  int T;         // 16-row x tiles (skinny)
  bool persist;  // persistent workgroups, one per CU (skinny)
  size_t lds;
  int grid;
};

static ProjLaunch plan_projection(const ProjArgs& a) {
  ProjLaunch l{};
  const int nstrips = a.Np / kStrip;
  if (a.M == 1) {
    l.gemv = true;
    l.g = gemv_plan(nstrips, a.G);
    l.lds = gemv_lds_bytes(a.K, l.g);
    l.grid = (nstrips + l.g.SP - 1) / l.g.SP;
    return l;
  }
  // the multi-row GEMV for M = 2 and 3, when its x staging fits (the
  // scaled x of all rows in LDS, within kRowsXMax 16-byte chunks per
  // thread).  Against the skinny kernel (one group of atoms in flight,
  // consecutive atoms overlapping) the whole 70B-shape step took 103.5 /
  // 106 / 121 / 122 us at M = 2 / 3 / 6 / 8 with it and 106 / 108.7 / 115 /
  // 112 without; with 4 atoms per wave in flight the 8B-shape step took
  // 45.4 / 49.9 / 51.8 us at M = 2 / 3 / 4 with it against 49.3 (M = 2, the
  // former 8) / 51.1 / 51.5 without, the 70B-shape step at M = 4 106.5
  // against 106.9 (alternating on one box).
  if (a.M <= 3) {
    const GemvPlan g = gemv_plan(nstrips, a.G);
    const int gpw_t = gemv_reg_groups(g, a.G);
    const size_t lds = gemv_rows_lds_bytes(a.K, a.M, g, gpw_t);
    const int xn = (a.M * (a.K / 8) + g.NW * 64 - 1) / (g.NW * 64);
    if (lds <= (size_t)kMaxLdsBytes && xn <= kRowsXMax) {
      l.gemv = true;
      l.rows = true;
      l.g = g;
      l.lds = lds;
      l.grid = (nstrips + g.SP - 1) / g.SP;
      return l;
    }
  }
  {
    l.T = a.M <= 16 ? 1 : 2;
    l.s = skinny_plan(nstrips, a.G, l.T, split_bytes_of(a));
    l.lds = l.s.SP ? skinny_lds_bytes(l.s.GPW, l.s.SP, l.T) : 0;
    const int ntiles = l.s.SP ? (nstrips + l.s.SP - 1) / l.s.SP * l.s.KS : 0;
    // more tiles than CUs at seven strips and one x tile: persistent
    // workgroups, one per CU
    l.persist = ntiles > kSkinnyMaxWorkgroups && l.s.SP == 7 && l.T == 1;
    l.grid = l.persist ? kSkinnyMaxWorkgroups : ntiles;
  }
  return l;
}

// The skinny instantiation that matches a plan: launched (launch == true)
// or only looked up.  Returns false when the library holds no kernel for
// the plan, so a plan without one is an error instead of a silent no-op.
// (Two x tiles with the persistent loop exceed the register file.)
template <int EPI>
static bool skinny_dispatch(const ProjArgs& a, const ProjLaunch& l, hipStream_t st, bool launch) {
  const SkinnyPlan& p = l.s;
#define I4D_SKINNY(SPV, TV, DV, PV)                                                                             \
  if (p.SP == SPV && l.T == TV && p.D == DV && l.persist == PV) {                                               \
    if (launch)                                                                                                 \
      hipLaunchKernelGGL((proj_skinny_kernel<EPI, SPV, TV, DV, PV>), dim3(l.grid), dim3(kSkinnyWaves * 64), l.lds, \
                         st, a, p);                                                                             \
    return true;                                                                                                \
  }
  I4D_SKINNY(7, 1, 1, true)
  I4D_SKINNY(1, 1, 2, false) I4D_SKINNY(2, 1, 2, false) I4D_SKINNY(3, 1, 2, false) I4D_SKINNY(4, 1, 1, false)
  I4D_SKINNY(5, 1, 1, false) I4D_SKINNY(7, 1, 1, false)
  I4D_SKINNY(1, 2, 2, false) I4D_SKINNY(2, 2, 1, false) I4D_SKINNY(3, 2, 1, false) I4D_SKINNY(4, 2, 1, false)
  I4D_SKINNY(5, 2, 1, false) I4D_SKINNY(7, 2, 1, false)
#undef I4D_SKINNY
  return false;
}

template <int EPI>
static bool launch_epi(const ProjArgs& a, hipStream_t st, bool launch) {
  const ProjLaunch l = plan_projection(a);
  if (l.gemv) {
    if (!launch) return true;  // launch_gemv(_rows) has a kernel for every plan
    if (l.rows) {
      if (l.g.NW == 16)
        launch_gemv_rows<EPI, 16>(a, l.g, l.lds, l.grid, st);
      else if (l.g.NW == 8)
        launch_gemv_rows<EPI, 8>(a, l.g, l.lds, l.grid, st);
      else
        launch_gemv_rows<EPI, 4>(a, l.g, l.lds, l.grid, st);
      return true;
    }
    if (l.g.NW == 16)
      launch_gemv<EPI, 16>(a, l.g, l.lds, l.grid, st);
    else if (l.g.NW == 8)
      launch_gemv<EPI, 8>(a, l.g, l.lds, l.grid, st);
    else
      launch_gemv<EPI, 4>(a, l.g, l.lds, l.grid, st);
    return true;
  }
  return skinny_dispatch<EPI>(a, l, st, launch);
}

static bool dispatch_epi(int epi, const ProjArgs& a, hipStream_t st, bool launch) {
  switch (epi) {
    case EPI_QKV: return launch_epi<EPI_QKV>(a, st, launch);
    case EPI_O: return launch_epi<EPI_O>(a, st, launch);
    case EPI_GU: return launch_epi<EPI_GU>(a, st, launch);
    case EPI_DOWN: return launch_epi<EPI_DOWN>(a, st, launch);
    default: return false;
  }
}

// shape limits of the kernels (message set when unsupported)
static i4d_status projection_fits(const ProjArgs& a, const ProjLaunch& l) {
  if (l.gemv) {
    // the multi-row plan is only chosen where its staging fits
    if (!l.rows && (l.lds > (size_t)kMaxLdsBytes || a.K > 4 * 8 * l.g.NW * 64))
      return fail(I4D_ERR_UNSUPPORTED, "K=%d too large for the M=1 kernel (LDS %zu bytes)", a.K, l.lds);
  } else if (l.s.SP == 0) {
    return fail(I4D_ERR_UNSUPPORTED, "K=%d too large for the M>1 kernel", a.K);
  }
  return ok();
}

i4d_status launch_projection(int epi, const ProjArgs& a, hipStream_t st) {
  if (epi < EPI_QKV || epi > EPI_DOWN) return fail(I4D_ERR_RANGE, "bad epilogue %d", epi);
  if (a.fmt == kFmtE4M3) return launch_projection_e4m3(epi, a, st);
  const ProjLaunch l = plan_projection(a);
  const i4d_status fit = projection_fits(a, l);
  if (fit != I4D_OK) return fit;
  if (!dispatch_epi(epi, a, st, true))
    return fail(I4D_ERR_UNSUPPORTED, "no projection kernel for the plan (SP %d, T %d, D %d, persistent %d)", l.s.SP,
                l.T, l.s.D, (int)l.persist);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(I4D_ERR_HIP, "projection launch: %s", hipGetErrorString(e));
  return ok();
}

i4d_status projection_plan_of(int epi, const ProjArgs& a, i4d_projection_plan* out) {
  const ProjLaunch l = plan_projection(a);
  *out = i4d_projection_plan{};
  out->kernel = l.gemv ? (l.rows ? 2 : 0) : 1;
  out->waves = l.gemv ? l.g.NW : kSkinnyWaves;
  out->strips_per_workgroup = l.gemv ? l.g.SP : l.s.SP;
  out->k_slices = l.gemv ? 1 : l.s.KS;
  out->depth = l.gemv ? 0 : l.s.D;
  out->persistent = l.persist ? 1 : 0;
  out->grid = l.grid;
  out->lds_bytes = l.lds;
  const i4d_status fit = projection_fits(a, l);
  if (fit != I4D_OK) return fit;
  out->instantiated = dispatch_epi(epi, a, nullptr, false) ? 1 : 0;
  return ok();
}

SplitNeed projection_split_need(int Np, int K, int M) {
  SplitNeed n{0, 0};
  if (M <= 1) return n;
  const int nstrips = Np / kStrip, G = K / kGroup;
  if ((size_t)M * K * 2 <= kSplitMinXBytes) return n;
  const SkinnyPlan p = skinny_plan(nstrips, G, M <= 16 ? 1 : 2, (size_t)-1);
  if (p.KS > 1) {
    const size_t nsets = (size_t)(nstrips + p.SP - 1) / p.SP;
    n.part_bytes = nsets * p.KS * split_block_floats(p.SP) * sizeof(float);
    n.counters = nsets;
  }
  return n;
}

}  // namespace i4d
