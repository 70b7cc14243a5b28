// gemv_rows.h - INT4 projection of 2..8 rows of x on the M = 1 weight
// stream (gfx950).
//
// The M = 1 GEMV puts the same x in all 16 rows of the MFMA's A operand.
// Here rows 0..M-1 of A hold rows 0..M-1 of x, so the four 16x16x32
// products of an atom give every row's dot with the atom's 16 weight rows
// at once: the weight stream, the nibble decode and the MFMA count are
// those of M = 1 ("how it differs": group scales applied after
// accumulation, the batch of 2..32 rows on matrix cores).  Lane (c, j)
// receives rows 4j + i (i = 0..3) of weight row c, so lanes j = 0, 1 hold
// the M <= 8 results.
//
// x enters as fp16 scaled per (row, 128-group) by a power of two 2^sh
// (max |x| 2^sh of the group in [2^12, 2^13)) and by 1/16 at the positions
// paired with a byte's high nibble, exactly as at M = 1; per (group, row)
// the code offset term -8 * 2^-24 * (sum of the scaled x) * 2^-sh and 2^-sh
// sit in LDS, read per atom by the lanes of the output rows.  The
// workgroup loads x once and converts every value once into LDS (rows
// padded by 16 bytes, so that reads of different rows hit different
// banks); with GPW > 0 each wave then copies its groups into registers
// (lane (r, j) supplies A row r, i.e. x row r) and the partial sums reuse
// that LDS; with GPW == 0 the MFMA operands are read from LDS.
#pragma once
#include <algorithm>

#include "gemv.h"

namespace i4d {

constexpr int kRowsMax = 8;

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// the groups of x per wave that the kernel keeps in registers for a plan
// (1, 2 or 4 when every wave owns exactly that many), else 0 (x in LDS)
inline int gemv_reg_groups(const GemvPlan& p, int G) {
  if (G % p.NW != 0) return 0;
  return (p.GPW == 1 || p.GPW == 2 || p.GPW == 4) ? p.GPW : 0;
}

// 16-byte chunks of x per thread in the workgroup's staging of x
constexpr int kRowsXMax = 8;

// LDS of the multi-row kernel: x~ [M][K + 8] fp16, with GPW > 0 shared with
// the partials [SP][NW][16][M] (x~ is in registers by then), else followed
// by them | (offset term, 2^-sh) [G][8] | tile [SP*16][M] | rho [8] | per
// (row, group) sums of squares [M][G]
constexpr int kRowsPad = 8;  // fp16 padding per row of x~
inline size_t gemv_rows_lds_bytes(int K, int M, const GemvPlan& p, int gpw_t) {
  const int G = K / kGroup;
  const size_t xb = (size_t)M * (K + kRowsPad) * 2, rb = (size_t)p.SP * p.NW * 16 * M * 4;
  size_t b = gpw_t > 0 ? std::max(xb, rb) : xb + rb;
  b += (size_t)G * kRowsMax * 8;
  b += (size_t)p.SP * 16 * M * 4;
  b += kRowsMax * 4;
  b += (size_t)M * G * 4;
  return b;
}

// power-of-two range scale of a group with maximum |x| = mx
__device__ __forceinline__ void rows_group_scale(float mx, float& sigma, float& unscale) {
  int ex = 0;
  if (mx > 0.f) frexpf(mx, &ex);
  const int sh = max(-100, min(100, 13 - ex));
  sigma = ldexpf(1.0f, sh);
  unscale = ldexpf(1.0f, -sh);
}

// 8 bf16 values -> fp16 scaled by sigma, and by 1/16 at e in {2, 3, 6, 7}
__device__ __forceinline__ u32x4_t rows_to_f16(const u32x4_t v, float sigma) {
  u32x4_t o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float f = (e & 1) ? sigma * 0.0625f : sigma;
    const f16x2_t h = {(_Float16)(bf16_lo(v[e]) * f), (_Float16)(bf16_hi(v[e]) * f)};
    o[e] = bitcast<uint32_t>(h);
  }
  return o;
}

template <int EPI, int NW, int U, int GPW, int XMAX>
__device__ __forceinline__ void gemv_rows_body(const ProjArgs& a, const GemvPlan& pl, const int strip0,
                                               const int ns, unsigned char* smem) {
  const int K = a.K, G = a.G, M = a.M;
  const int SP = pl.SP;
  const int GW = GPW > 0 ? GPW : pl.GPW;
  const int KP = K + kRowsPad;  // row pitch of x~ in LDS (fp16)
  const size_t xb = (size_t)M * KP * 2, rb = (size_t)SP * NW * 16 * M * 4;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);  // [M][KP] fp16
  float* red = reinterpret_cast<float*>(smem + (GPW > 0 ? 0 : xb));  // [SP][NW][16][M]
  size_t off = GPW > 0 ? (xb > rb ? xb : rb) : xb + rb;
  float2* Xs = reinterpret_cast<float2*>(smem + off);  // (offset term, 2^-sh) [G][kRowsMax]
  off += (size_t)G * kRowsMax * 8;
  float* ot = reinterpret_cast<float*>(smem + off);  // [SP*16][M]
  off += (size_t)SP * 16 * M * 4;
  float* rho = reinterpret_cast<float*>(smem + off);  // [kRowsMax]
  off += kRowsMax * 4;
  float* gsq = reinterpret_cast<float*>(smem + off);  // [M][G] sums of squares

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int nstrips = a.Np / kStrip;
  const int g0 = wave * GW;                 // first group of this wave
  const int gpw = max(0, min(GW, G - g0));  // groups of this wave
  const int n = ns * gpw;                   // atoms of this wave
  const int npad = ((max(n, 1) + U - 1) / U) * U;
  constexpr int GR = GPW > 0 ? GPW : 1;
  static_assert(U % GR == 0, "the ring must hold whole strips");
  const int xrow = min(r, M - 1);  // the x row this lane supplies as A row r

  // 1. x: the thread's 16-byte chunks of all rows (clamped, so every thread
  // issues the same number of loads), before the weights
  u32x4_t xv[XMAX];
  const int nchunk = M * (K / 8);
  const int xn = (nchunk + NW * 64 - 1) / (NW * 64);  // <= XMAX (host-checked)
#pragma unroll
  for (int q = 0; q < XMAX; ++q)
    if (q < xn) xv[q] = load16(a.x + (size_t)min(tid + q * NW * 64, nchunk - 1) * 8);

  // 2. the first U atoms of the weight stream with their scales (the
  // cursor walks strip by strip through the wave's groups)
  int rs = 0, rg = 0;
  auto next_atom = [&](const uint8_t*& cp, const uint16_t*& sp) {
    const int t = min(strip0 + rs, nstrips - 1);
    const int g = min(g0 + rg, G - 1);
    cp = a.codes + ((size_t)t * G + g) * kAtomBytes + (size_t)lane * 16;
    sp = a.scales + ((size_t)t * G + g) * kStrip + r;
    if (rs < ns - 1 || rg < gpw - 1) {
      if (++rg >= gpw) {
        rg = 0;
        ++rs;
      }
    }
  };
  u32x4_t ring[U];
  uint16_t sring[U];
  int fill_round = 0;
  const int last_strip = min(strip0 + max(ns, 1) - 1, nstrips - 1);
  const uint32_t lane_off = (uint32_t)lane * 16;
  auto fill = [&](const int k) {
    const uint8_t* cp;
    const uint16_t* sp;
    if (GPW > 0) {
      const int t = min(strip0 + fill_round * (U / GR) + k / GR, last_strip);
      const size_t atom = (size_t)t * G + min(g0 + (k % GR), G - 1);
      cp = a.codes + atom * kAtomBytes + lane_off;
      sp = a.scales + atom * kStrip + r;
      if (k == U - 1) ++fill_round;
    } else {
      next_atom(cp, sp);
    }
    ring[k] = load16_stream(cp);
    sring[k] = *sp;
  };
  // in the loop's order (each slot's data, then its scale): the loop's waits
  // count loads from the loop entry too, and a different order there would
  // shorten them for every iteration
#pragma unroll
  for (int k = 0; k < U; ++k) {
    fill(k);
    __builtin_amdgcn_sched_barrier(0);
  }

  // 3. scaled fp16 x.  Chunk c (16 per group of a row) sits in lane c % 16
  // of a 16-lane row: the group's maximum, sum of squares and scaled sum
  // are 16-lane reductions.
  constexpr float kOffset = -8.0f / 16777216.0f;
  const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
  const f16x2_t sixteen = {(_Float16)16.0f, (_Float16)16.0f};
#pragma unroll
  for (int q = 0; q < XMAX; ++q) {
    if (q < xn) {
      const int cidx = tid + q * NW * 64;
      u16x2_t mb = {0, 0};
      float sqc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = xv[q][e];
        sqc = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(w), bitcast<bf16x2_t>(w), sqc, false);
        mb = __builtin_elementwise_max(mb, bitcast<u16x2_t>(w & 0x7FFF7FFFu));
      }
      // bf16 magnitudes order like unsigned integers
      float mx = __uint_as_float((uint32_t)max(mb[0], mb[1]) << 16);
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) {
        mx = fmaxf(mx, lane_xor(mx, o, lane));
        sqc += lane_xor(sqc, o, lane);
      }
      float sigma, unscale;
      rows_group_scale(mx, sigma, unscale);
      const u32x4_t h = rows_to_f16(xv[q], sigma);
      float cs = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        cs = __builtin_amdgcn_fdot2(bitcast<f16x2_t>(h[e]), (e & 1) ? sixteen : one, cs, false);
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) cs += lane_xor(cs, o, lane);
      if (cidx < nchunk) {  // whole groups: K / 8 is a multiple of 16
        const int m = cidx / (K / 8), k8 = cidx % (K / 8), g = k8 / 16;
        *reinterpret_cast<u32x4_t*>(xs + (size_t)m * KP + 8 * k8) = h;
        if ((lane & 15) == 0) {
          Xs[g * kRowsMax + m] = make_float2(cs * kOffset * unscale, unscale);
          gsq[m * G + g] = sqc;
        }
      }
    }
  }
  lds_barrier();
  // rho: wave w sums rows w, w + NW, ... (read only after later barriers)
  if (needs_rho<EPI>()) {
    for (int m = wave; m < M; m += NW) {
      float sq = 0.f;
      for (int g = lane; g < G; g += 64) sq += gsq[m * G + g];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) sq += lane_xor(sq, o, lane);
      if (lane == 0) rho[m] = 1.0f / sqrtf(sq / (float)K + a.eps);
    }
  } else if (tid < M) {
    rho[tid] = 1.0f;
  }
  // GPW > 0: the wave's groups of its A row into registers; the partials
  // then reuse the LDS of x~
  u32x4_t xr[GR][4];
  if (GPW > 0) {
    const u32x4_t* xl = reinterpret_cast<const u32x4_t*>(xs + (size_t)xrow * KP);
#pragma unroll
    for (int gi = 0; gi < GR; ++gi)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) xr[gi][kb] = xl[(128 * (g0 + gi) + 32 * kb + 8 * j) / 8];
    lds_barrier();
  }

  // 4. stream: consume atom i from the ring, then refill its slot with
  // atom i + U.  Per atom four MFMAs (x rows as A, decoded codes as B);
  // lane (c, j) applies the offset terms and 2^-sh of rows 4j + i and the
  // scale of weight row c.  Lanes j >= 2 compute rows past 8 (unused) and read
  // the terms of rows 4 .. 7.
  const float2* Xj = Xs + 4 * min(j, 1);
  float part[4] = {0.f, 0.f, 0.f, 0.f};
  int sl = 0, gi_rt = 0;
  auto consume = [&](const u32x4_t w, const uint16_t sbits, int i, int k) {
    if (i < n) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      int g;
      if (GPW > 0) {
        const int gi = k % GR;
        g = g0 + gi;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8_t>(xr[gi][kb]), dword_to_f16x8_sub(w[kb]),
                                                       acc, 0, 0, 0);
      } else {
        g = g0 + gi_rt;
        const u32x4_t* xl = reinterpret_cast<const u32x4_t*>(xs + (size_t)xrow * KP);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8_t>(xl[(128 * g + 32 * kb + 8 * j) / 8]),
                                                       dword_to_f16x8_sub(w[kb]), acc, 0, 0, 0);
      }
      const f32x4_t* xp = reinterpret_cast<const f32x4_t*>(Xj + g * kRowsMax);
      const f32x4_t t01 = xp[0], t23 = xp[1];  // (offset, 2^-sh) of rows 4j, 4j+1 | 4j+2, 4j+3
      const float sc = f16_bits_to_f32(sbits);
      part[0] = fmaf(sc, fmaf(acc[0], t01[1], t01[0]), part[0]);
      part[1] = fmaf(sc, fmaf(acc[1], t01[3], t01[2]), part[1]);
      part[2] = fmaf(sc, fmaf(acc[2], t23[1], t23[0]), part[2]);
      part[3] = fmaf(sc, fmaf(acc[3], t23[3], t23[2]), part[3]);
      const bool last_of_strip = (GPW > 0) ? (k % GR == GR - 1) : (gi_rt == gpw - 1);
      if (last_of_strip) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int row = 4 * j + ii;
          if (row < M) red[(((size_t)sl * NW + wave) * 16 + r) * M + row] = part[ii];
          part[ii] = 0.f;
        }
        ++sl;
      }
      if (GPW == 0) gi_rt = last_of_strip ? 0 : gi_rt + 1;
    }
  };
  int i0 = 0;
  for (; i0 + U < npad; i0 += U) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      consume(ring[k], sring[k], i0 + k, k);
      fill(k);
    }
  }
#pragma unroll
  for (int k = 0; k < U; ++k) consume(ring[k], sring[k], i0 + k, k);
  // waves without a group range leave zero partials
  for (int s2 = sl; s2 < ns; ++s2)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int row = 4 * j + ii;
      if (row < M) red[(((size_t)s2 * NW + wave) * 16 + r) * M + row] = 0.f;
    }
  lds_barrier();

  // 5. reduce over the waves; undo the 2^-24 of the code operand; epilogue
  // (rho per row computed with the staging)
  for (int idx = tid; idx < ns * 16 * M; idx += NW * 64) {
    const int s2 = idx / (16 * M), rem = idx - s2 * 16 * M;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[((size_t)s2 * NW + w) * 16 * M + rem];
    ot[idx] = v * 16777216.0f;
  }
  lds_barrier();
  run_epilogue<EPI>(a, strip0, ns, ot, rho);
}

}  // namespace i4d
