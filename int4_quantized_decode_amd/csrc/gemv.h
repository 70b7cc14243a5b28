// gemv.h - M = 1 INT4 projection (one row of x, MFMA dot products) as a
// device function, shared by the stand-alone projection kernels and the
// one-launch decode step.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "coherent.h"
#include "device_common.h"
#include "i4d_internal.h"
#include "proj.h"

namespace i4d {

template <int EPI>
__host__ __device__ __forceinline__ constexpr bool needs_rho() {
  return EPI == EPI_QKV || EPI == EPI_GU;
}

// the wait hook of a stage whose input is ready at entry
struct NoWait {
  __device__ void operator()() const {}
};

template <bool COH>
__device__ __forceinline__ void st_out(float* p, float v) {
  if (COH) st_coh(p, v); else *p = v;
}
template <bool COH>
__device__ __forceinline__ void st_out(uint16_t* p, uint16_t v) {
  if (COH) st_coh(p, v); else *p = v;
}

// RoPE, rotate-half pair (c0, c0 + hd/2) at position pos: angle pos *
// theta^(-2 c0 / hd) in fp64 (the frequency as (theta^(-2/hd))^c0 by binary
// powering of the host's fp64 ratio), reduced to [-pi, pi], then fp32 sin/cos
__device__ __forceinline__ void rope_angle(double ratio, int pos, int c0, float& cs, float& sn) {
  double freq = 1.0, base = ratio;
  for (int e = c0; e; e >>= 1) {
    if (e & 1) freq *= base;
    base *= base;
  }
  const double ang = (double)pos * freq;
  const double k2pi = rint(ang * 0.15915494309189535);
  double red = fma(-k2pi, 6.283185307179586, ang);
  red = fma(-k2pi, 2.4492935982947064e-16, red);
  sincosf((float)red, &sn, &cs);
}

// Inputs of the epilogue that do not depend on the weight stream, for the
// thread's first output (idx = threadIdx.x): the residual of O and down, the
// RoPE rotation of QKV.  The M = 1 kernel reads or computes them ahead of
// the stream, so that their latency is not added after it.
struct EpiPre {
  float res, cs, sn;
  bool valid;
};

// Epilogue from the LDS tile ot[row][M] (rows of strips strip0 .. strip0+S-1).
// COH: outputs consumed inside the same launch are stored agent-coherently
// and the in-launch residual (h, down projection) is loaded the same way.
template <int EPI, bool COH = false>
__device__ void run_epilogue(const ProjArgs& a, int strip0, int S, const float* ot, const float* rho,
                             const EpiPre* pre = nullptr) {
  const int M = a.M;
  const int nthreads = blockDim.x;
  if (EPI == EPI_QKV || EPI == EPI_GU) {
    for (int idx = threadIdx.x; idx < S * 8 * M; idx += nthreads) {
      const bool use_pre = pre && pre->valid && idx == (int)threadIdx.x;
      const int m = idx % M, pi = idx / M, s = pi / 8, i = pi % 8;
      const int t = strip0 + s;
      if (t * kStrip >= a.Np) continue;
      float y0 = ot[(s * 16 + i) * M + m] * rho[m];
      float y1 = ot[(s * 16 + 8 + i) * M + m] * rho[m];
      if (EPI == EPI_GU) {
        const int f = 8 * t + i;
        const float silu = y0 / (1.0f + expf(-y0));
        st_out<COH>(&a.a_out[(size_t)m * (a.Np / 2) + f], f32_to_bf16(silu * y1));
      } else {
        const int per_head = a.hd / kStrip;
        const int head = t / per_head, sp = t % per_head;
        const int c0 = 8 * sp + i, c1 = c0 + a.hd / 2;
        if (head < a.n_q + a.n_kv) {
          float sn_f, c;
          if (use_pre) {
            c = pre->cs;
            sn_f = pre->sn;
          } else {
            rope_angle(a.rope_ratio, a.ctx_len[m] - 1, c0, c, sn_f);
          }
          const float r0 = y0 * c - y1 * sn_f;
          const float r1 = y1 * c + y0 * sn_f;
          y0 = r0;
          y1 = r1;
        }
        // COH (one-launch step, M = 1): the attention units read the
        // flagged copies; the plain ones are the step's visible outputs
        if (head < a.n_q) {
          float* q = a.q_out + ((size_t)m * a.n_q + head) * a.hd;
          st_out<COH>(&q[c0], y0);
          st_out<COH>(&q[c1], y1);
          if (COH) {
            uint64_t* ql = a.q_ll + (size_t)head * a.hd;
            st_flag(&ql[c0], __float_as_uint(y0), *a.epoch + 1u);
            st_flag(&ql[c1], __float_as_uint(y1), *a.epoch + 1u);
          }
        } else {
          const bool is_k = head < a.n_q + a.n_kv;
          const int kvh = head - a.n_q - (is_k ? 0 : a.n_kv);
          uint16_t* kv = (is_k ? a.k_out : a.v_out) + ((size_t)m * a.n_kv + kvh) * a.hd;
          const uint16_t b0 = f32_to_bf16(y0), b1 = f32_to_bf16(y1);
          st_out<COH>(&kv[c0], b0);
          st_out<COH>(&kv[c1], b1);
          if (COH) {
            uint64_t* kl = (is_k ? a.k_ll : a.v_ll) + (size_t)kvh * a.hd;
            st_flag(&kl[c0], b0, *a.epoch + 1u);
            st_flag(&kl[c1], b1, *a.epoch + 1u);
          }
        }
      }
    }
  } else {
    for (int idx = threadIdx.x; idx < S * 16 * M; idx += nthreads) {
      const bool use_pre = pre && pre->valid && idx == (int)threadIdx.x;
      const int m = idx % M, row = idx / M;
      const int n = strip0 * kStrip + row;
      if (n >= a.Np) continue;
      const float y = ot[row * M + m];
      const size_t o = (size_t)m * a.Np + n;
      if (EPI == EPI_O) {
        const float h = (use_pre ? pre->res : bf16_to_f32(a.resid_bf16[o])) + y;
        st_out<COH>(&a.h_f32[o], h);
        st_out<COH>(&a.h_bf16[o], f32_to_bf16(h));
      } else {
        const float res = use_pre ? pre->res : (COH ? ld_coh(&a.resid_f32[o]) : a.resid_f32[o]);
        a.out_bf16[o] = f32_to_bf16(res + y);
      }
    }
  }
}

// Launch shape of the M = 1 kernel: NW waves, SP strips per workgroup, GPW
// = G / NW groups per wave (the K range is split across the waves).
struct GemvPlan {
  int NW, SP, GPW;
};

// LDS: x [K] fp16 (GPW == 0) | per group (offset term, 2^-shift) [G] |
// partials [SP][NW][16] | tile [SP*16] | per-wave sums of squares [NW]
inline size_t gemv_lds_bytes(int K, const GemvPlan& p) {
  return (size_t)K * 2 + (size_t)(K / kGroup) * 8 + (size_t)p.SP * p.NW * 16 * 4 +
         (size_t)p.SP * 16 * 4 + (size_t)p.NW * 4;
}

// sum of the x values that 16 fp16 words of one group quarter represent
// (the factor 16 undoes the 1/16 at e in {2, 3, 6, 7})
__device__ __forceinline__ float quarter_sum(const u32x4_t (&xk)[4]) {
  const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
  const f16x2_t sixteen = {(_Float16)16.0f, (_Float16)16.0f};
  float s = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      s = __builtin_amdgcn_fdot2(bitcast<f16x2_t>(xk[kb][q]), (q & 1) ? sixteen : one, s, false);
  return s;
}

// One wave streams its atoms (strip s of the workgroup, group g of its K
// range) through a ring of U outstanding 16-byte loads per lane (plus the
// 2-byte scale of each atom).  The atom sequence is padded to a multiple of
// U with repeats of its last atom (L2 hits, no HBM traffic), so every round
// issues exactly U loads and the compiler can wait on exact counts.
//
// x enters the MFMA as fp16, per 128-group g scaled by a power of two
// (max |x_g| 2^sh_g in [2^12, 2^13), so the conversion from bf16 is exact
// for every value above 2^-23 of the group maximum) and by 1/16 at the
// positions paired with the high nibble of a byte; the group's scale comes
// from a reduction over the 16 lanes that stage it, so one workgroup
// barrier separates the x loads from the stream.  With GPW > 0 (compile
// time, a divisor of U) each wave then keeps its GPW groups of x in
// registers; GPW == 0 reads x from LDS for every atom.
//
// The body serves the stand-alone kernel and the one-launch decode step
// (COH = true): there `wait_input` blocks until the producers of x are done
// (the last wave polls, from lane 0), then x is read agent-coherently, then
// the ring is requested (with PRE: before the wait, for a wait long enough
// to cover the atoms' latency); the outputs are stored agent-coherently.
// `strip0`, `ns`: the strips of this workgroup (ns <= pl.SP).
template <int EPI, int NW, int U, int GPW, bool COH, bool PRE = false, typename Wait>
__device__ __forceinline__ void gemv_body(const ProjArgs& a, const GemvPlan& pl, const int strip0,
                                          const int ns, unsigned char* smem, Wait&& wait_input) {
  const int K = a.K, G = a.G;
  const int SP = pl.SP;
  const int GW = GPW > 0 ? GPW : pl.GPW;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                  // [K] fp16
  float2* Xs = reinterpret_cast<float2*>(smem + (size_t)K * 2);      // [G]
  float* red = reinterpret_cast<float*>(Xs + G);                     // [SP][NW][16]
  float* ot = red + (size_t)SP * NW * 16;                            // [SP*16]
  float* ssq = ot + SP * 16;                                         // [NW]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int r = lane & 15, j = lane >> 4;
  const int nstrips = a.Np / kStrip;
  const int g0 = wave * GW;                   // first group of this wave
  const int gpw = max(0, min(GW, G - g0));    // groups of this wave
  const int n = ns * gpw;                     // atoms of this wave
  const int npad = ((max(n, 1) + U - 1) / U) * U;
  constexpr int GR = GPW > 0 ? GPW : 1;
  static_assert(U % GR == 0, "the ring must hold whole strips");

  // 1. x: the loads of this thread's 16-byte chunks (clamped, so every
  // thread issues the same number of loads).  Stand-alone: issued first, so
  // that every wave's x enters the memory pipeline before any weight load.
  // One-launch step: issued after the producers are done.
  constexpr int XMAX = 4;  // K <= XMAX * 8 * NW * 64 (host-checked)
  const int xn = (K / 8 + NW * 64 - 1) / (NW * 64);  // chunks per thread (uniform)
  u32x4_t xv[XMAX];
  auto load_x = [&]() {
#pragma unroll
    for (int q = 0; q < XMAX; ++q) {
      if (q < xn) {
        const int cidx = min(tid + q * NW * 64, K / 8 - 1);
        xv[q] = COH ? ld_coh16(a.x, (uint32_t)cidx * 16, (uint32_t)K * 2) : load16(a.x + (size_t)cidx * 8);
      }
    }
  };
  constexpr bool X_FIRST = !COH || std::is_same<std::decay_t<Wait>, NoWait>::value;
  // the epilogue's inputs of this thread's output (M = 1: output tid),
  // requested behind x: the residual, or the position for RoPE
  EpiPre pre = {0.f, 1.f, 0.f, false};
  int rope_pos = 0;
  auto load_pre = [&]() {
    if (a.M != 1) return;
    if (EPI == EPI_O || EPI == EPI_DOWN) {
      const int n = strip0 * kStrip + tid;
      if (tid < ns * kStrip && n < a.Np) {
        if (EPI == EPI_O) pre.res = bf16_to_f32(a.resid_bf16[n]);
        else pre.res = COH ? ld_coh(&a.resid_f32[n]) : a.resid_f32[n];
        pre.valid = true;
      }
    } else if (EPI == EPI_QKV && tid < ns * 8) {
      rope_pos = a.ctx_len[0] - 1;
      pre.valid = true;
    }
  };
  if (X_FIRST) {
    load_x();
    load_pre();
    lds_barrier();
  }

  // 2. the first U atoms of the weight stream, each with its scale (lane r:
  // row r of the atom's strip; scales are [strip][group][row], so a
  // 2-byte load per atom).  The refill cursor (rs, rg) walks strip by strip
  // through the wave's groups and stops on the last atom, which pads the
  // sequence.
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
  // GPW > 0: every wave has GR groups of each strip (or none), so slot k
  // always holds group k % GR of strip (round * U / GR + k / GR): one
  // clamped strip index and one scalar base per strip and round (the lane
  // offsets are fixed vector registers), no cursor arithmetic per atom
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
  // In the one-launch step the atoms are requested only after the wait and
  // the x loads: a wave's loads complete in order, so atoms requested
  // before would delay the polls and x behind them (measured slower).
  if (X_FIRST) {
#pragma unroll
    for (int k = 0; k < U; ++k) fill(k);
  }
  if (!X_FIRST) {
    if (PRE) {
#pragma unroll
      for (int k = 0; k < U; ++k) fill(k);
    }
    wait_input();
    load_x();
    load_pre();
    if (!PRE) {
#pragma unroll
      for (int k = 0; k < U; ++k) fill(k);
    }
  }

  // 3. fp16 x per group g, scaled by a power of two 2^sh_g (max|x_g| 2^sh_g
  // in [2^12, 2^13), so bf16 -> fp16 is exact for every value above 2^-23
  // of the group maximum) and by 1/16 at e in {2,3,6,7}; the group result
  // is scaled back by 2^-sh_g.  Per group: the code offset term
  // -8 * 2^-24 * (sum of the group's x) * 2^-sh_g and 2^-sh_g.  For QKV and
  // gate/up also the sum of squares of x (rho).
  constexpr float kOffset = -8.0f / 16777216.0f;
  auto group_scale = [](float mx, float& sigma, float& unscale) {
    int ex = 0;
    if (mx > 0.f) frexpf(mx, &ex);
    const int sh = max(-100, min(100, 13 - ex));
    sigma = ldexpf(1.0f, sh);
    unscale = ldexpf(1.0f, -sh);
  };
  auto to_f16 = [](const u32x4_t v, float sigma) {
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float f = (e & 1) ? sigma * 0.0625f : sigma;
      const f16x2_t h = {(_Float16)(bf16_lo(v[e]) * f), (_Float16)(bf16_hi(v[e]) * f)};
      o[e] = bitcast<uint32_t>(h);
    }
    return o;
  };
  const u32x4_t* xl = reinterpret_cast<const u32x4_t*>(xs);
  u32x4_t xr[GR][4];
  float xc[GR], xf[GR];
  float sq = 0.f;
  {
    // chunk c (16 per group) sits in lane c % 16 of a 16-lane row, so the
    // group's maximum and sum are row reductions
#pragma unroll
    for (int q = 0; q < XMAX; ++q) {
      const int cidx = tid + q * NW * 64;
      if (q < xn) {
        const bool valid = cidx < K / 8;  // whole groups: K is a multiple of 128
        float mx = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = bf16_lo(xv[q][e]), hi = bf16_hi(xv[q][e]);
          if (needs_rho<EPI>() && valid) {
            sq = fmaf(lo, lo, sq);
            sq = fmaf(hi, hi, sq);
          }
          mx = fmaxf(mx, fmaxf(fabsf(lo), fabsf(hi)));
        }
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) mx = fmaxf(mx, lane_xor(mx, o, lane));
        float sigma, unscale;
        group_scale(mx, sigma, unscale);
        const u32x4_t h = to_f16(xv[q], sigma);
        const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
        const f16x2_t sixteen = {(_Float16)16.0f, (_Float16)16.0f};
        float cs = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          cs = __builtin_amdgcn_fdot2(bitcast<f16x2_t>(h[e]), (e & 1) ? sixteen : one, cs, false);
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) cs += lane_xor(cs, o, lane);
        if (valid) {
          reinterpret_cast<u32x4_t*>(xs)[cidx] = h;
          if ((lane & 15) == 0) Xs[cidx >> 4] = make_float2(cs * kOffset * unscale, unscale);
        }
      }
    }
    if (needs_rho<EPI>()) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) sq += lane_xor(sq, o, lane);
      if (lane == 0) ssq[wave] = sq;
    }
    lds_barrier();
  }
  // the wave's own groups of x in registers
  if (GPW > 0) {
#pragma unroll
    for (int gi = 0; gi < GR; ++gi) {
      const int g = min(g0 + gi, G - 1);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) xr[gi][kb] = xl[(128 * g + 32 * kb + 8 * j) / 8];
      const float2 t = Xs[g];
      xc[gi] = t.x;
      xf[gi] = t.y;
    }
  }
  // RoPE rotation of this thread's output pair while the atoms are in flight
  if (EPI == EPI_QKV && pre.valid) {
    const int t = strip0 + tid / 8, i = tid % 8;
    const int per_head = a.hd / kStrip;
    const int head = t / per_head, sp = t % per_head;
    if (t < nstrips && head < a.n_q + a.n_kv) rope_angle(a.rope_ratio, rope_pos, 8 * sp + i, pre.cs, pre.sn);
  }

  // 6. stream: consume atom i from the ring, then refill its slot with atom
  // i + U (the loaded registers stay in place across iterations).  Per
  // atom, four MFMAs 16x16x32 with x in every row of A (lane (r, j) holds
  // the same x quarter j for any r) and the decoded codes as B (column r =
  // atom row r): every lane gets the whole 128-term dot of its row r,
  // scaled by 2^-24 and by the group's 2^sh; the code offset and 2^-sh
  // enter as one FMA per atom.
  float part = 0.f;
  int sl = 0, gi_rt = 0;  // strip and group of the atom being consumed (GPW == 0)
  auto consume = [&](const u32x4_t w, const uint16_t sbits, int i, int k) {
    if (i < n) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      if (GPW > 0) {
        const int gi = k % GR;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8_t>(xr[gi][kb]), dword_to_f16x8_sub(w[kb]),
                                                       acc, 0, 0, 0);
      } else {
        const int g = g0 + gi_rt;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8_t>(xl[(128 * g + 32 * kb + 8 * j) / 8]),
                                                       dword_to_f16x8_sub(w[kb]), acc, 0, 0, 0);
      }
      float y;
      if (GPW > 0) {
        const int gi = k % GR;
        y = fmaf(acc[0], xf[gi], xc[gi]);
      } else {
        const float2 t = Xs[g0 + gi_rt];
        y = fmaf(acc[0], t.y, t.x);
      }
      part = fmaf(f16_bits_to_f32(sbits), y, part);
      const bool last_of_strip = (GPW > 0) ? (k % GR == GR - 1) : (gi_rt == gpw - 1);
      if (last_of_strip) {
        if (j == 0) red[((size_t)sl * NW + wave) * 16 + r] = part;
        part = 0.f;
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
      // the refill is issued at raised wave priority, ahead of the other
      // waves' MFMAs (one-launch step 37.46 -> 37.33 us, alternating on one
      // box)
      __builtin_amdgcn_s_setprio(2);
      fill(k);
      __builtin_amdgcn_s_setprio(0);
    }
  }
#pragma unroll
  for (int k = 0; k < U; ++k) consume(ring[k], sring[k], i0 + k, k);
  // waves without a group range leave zero partials
  if (j == 0)
    for (int s2 = sl; s2 < ns; ++s2) red[((size_t)s2 * NW + wave) * 16 + r] = 0.f;
  lds_barrier();

  // 7. reduce over the waves; undo the 2^-24 of the code operand; epilogue
  if (tid < ns * 16) {
    const int s2 = tid >> 4, rr = tid & 15;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[((size_t)s2 * NW + w) * 16 + rr];
    ot[tid] = v * 16777216.0f;
  }
  if (needs_rho<EPI>() && tid == 0) {
    float t = 0.f;
    for (int w = 0; w < NW; ++w) t += ssq[w];
    ssq[0] = 1.0f / sqrtf(t / (float)K + a.eps);
  }
  lds_barrier();
  float one = 1.0f;
  run_epilogue<EPI, COH>(a, strip0, ns, ot, needs_rho<EPI>() ? &ssq[0] : &one, &pre);
}

}  // namespace i4d
