// proj.hip - INT4 projection kernels (gfx950): QKV, O, gate/up, down.
//
// y[m][n] = sum_g s[n][g] * sum_{k in g} (u[n][k] - 8) * x[m][k]
// ("how it differs": group scales applied after accumulation), computed as
// sum_g s[n][g] * (A[n][g] - 136 * X[m][g]) where A accumulates
// (128 + u) * x from the bf16 magic-exponent decode of each nibble and X is
// the group sum of x; the per-group scale and the 136 correction are applied
// once per group after the 128-wide accumulation.
//
// M = 1: register-streaming VALU GEMV.  Each 64-lane wave streams 1 KiB
//   atoms (16 rows x 128 k, one 16-byte load per lane) and accumulates with
//   v_dot2_f32_bf16 against x staged in LDS.
// M = 2..32: skinny GEMM on bf16 MFMA 16x16x32.  The atom lane layout is the
//   A operand; x[m] rows are the B operand read straight from global memory;
//   group sums of x and the RMSNorm sum of squares come from two extra MFMAs
//   (ones . x and x . x^T diagonal) so no VALU work is spent on them.
//
// Both kernels split K across the waves of a workgroup (interleaved groups),
// reduce in LDS and run the epilogue once per output from an LDS tile:
//   QKV : rho1 (from the staged input), RoPE on q/k pairs, q fp32, k/v bf16
//   O   : h = x + y (fp32 and bf16 copies)
//   GU  : rho2, a = silu(gate) * up (bf16)
//   DOWN: out = h + y (bf16)
#include <math.h>

#include "device_common.h"
#include "i4d_internal.h"
#include "proj.h"

namespace i4d {

constexpr int kMaxLdsBytes = 160 * 1024;

// LDS of the M = 1 kernel: x [K] bf16, group sums [G][4], reduction
// [NW][S*16], output tile [S*16], per-wave sums of squares + rho
static inline size_t gemv_lds_bytes(int K, int S, int NW) {
  return (size_t)K * 2 + (size_t)(K / kGroup) * 16 + (size_t)(NW * S * 16 + S * 16 + NW + 1) * 4;
}

template <int EPI>
__device__ __forceinline__ bool needs_rho() {
  return EPI == EPI_QKV || EPI == EPI_GU;
}

// Epilogue from the LDS tile ot[row][M] (rows of strips strip0 .. strip0+S-1)
template <int EPI>
__device__ void run_epilogue(const ProjArgs& a, int strip0, int S, const float* ot, const float* rho) {
  const int M = a.M;
  const int nthreads = blockDim.x;
  if (EPI == EPI_QKV || EPI == EPI_GU) {
    for (int idx = threadIdx.x; idx < S * 8 * M; idx += nthreads) {
      const int m = idx % M, pi = idx / M, s = pi / 8, i = pi % 8;
      const int t = strip0 + s;
      if (t * kStrip >= a.Np) continue;
      float y0 = ot[(s * 16 + i) * M + m] * rho[m];
      float y1 = ot[(s * 16 + 8 + i) * M + m] * rho[m];
      if (EPI == EPI_GU) {
        const int f = 8 * t + i;
        const float silu = y0 / (1.0f + expf(-y0));
        a.a_out[(size_t)m * (a.Np / 2) + f] = f32_to_bf16(silu * y1);
      } else {
        const int per_head = a.hd / kStrip;
        const int head = t / per_head, sp = t % per_head;
        const int c0 = 8 * sp + i, c1 = c0 + a.hd / 2;
        if (head < a.n_q + a.n_kv) {
          // RoPE, rotate-half pair (c0, c0 + hd/2) at position ctx_len - 1:
          // angle pos * theta^(-2 c0 / hd) in fp64, reduced to [-pi, pi],
          // then fp32 sin/cos
          const double pos = (double)(a.ctx_len[m] - 1);
          const double ang = pos * exp2(-(2.0 * (double)c0 / (double)a.hd) * log2((double)a.theta));
          const double k2pi = rint(ang * 0.15915494309189535);
          double red = fma(-k2pi, 6.283185307179586, ang);
          red = fma(-k2pi, 2.4492935982947064e-16, red);
          float sn_f, c;
          sincosf((float)red, &sn_f, &c);
          const float r0 = y0 * c - y1 * sn_f;
          const float r1 = y1 * c + y0 * sn_f;
          y0 = r0;
          y1 = r1;
        }
        if (head < a.n_q) {
          float* q = a.q_out + ((size_t)m * a.n_q + head) * a.hd;
          q[c0] = y0;
          q[c1] = y1;
        } else if (head < a.n_q + a.n_kv) {
          uint16_t* k = a.k_out + ((size_t)m * a.n_kv + (head - a.n_q)) * a.hd;
          k[c0] = f32_to_bf16(y0);
          k[c1] = f32_to_bf16(y1);
        } else {
          uint16_t* v = a.v_out + ((size_t)m * a.n_kv + (head - a.n_q - a.n_kv)) * a.hd;
          v[c0] = f32_to_bf16(y0);
          v[c1] = f32_to_bf16(y1);
        }
      }
    }
  } else {
    for (int idx = threadIdx.x; idx < S * 16 * M; idx += nthreads) {
      const int m = idx % M, row = idx / M;
      const int n = strip0 * kStrip + row;
      if (n >= a.Np) continue;
      const float y = ot[row * M + m];
      const size_t o = (size_t)m * a.Np + n;
      if (EPI == EPI_O) {
        const float h = bf16_to_f32(a.resid_bf16[o]) + y;
        a.h_f32[o] = h;
        a.h_bf16[o] = f32_to_bf16(h);
      } else {
        a.out_bf16[o] = f32_to_bf16(a.resid_f32[o] + y);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// M = 1: VALU GEMV
// ---------------------------------------------------------------------------

// Workgroup barrier that waits for LDS traffic only: weight loads stay in
// flight across it (__syncthreads would also drain every outstanding global
// load of the wave).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Launch shape of the M = 1 kernel: NW waves, SP strips per workgroup, GPW
// = G / NW groups per wave (the K range is split across the waves).
struct GemvPlan {
  int NW, SP, GPW;
};

// LDS: x [K] fp16 | group sums [G][4] | partials [SP][NW][16] | tile [SP*16]
// | per-wave sums of squares [NW] | per-wave max |x| [NW]
static inline size_t gemv_lds_bytes(int K, const GemvPlan& p) {
  return (size_t)K * 2 + (size_t)(K / kGroup) * 16 + (size_t)p.SP * p.NW * 16 * 4 +
         (size_t)p.SP * 16 * 4 + (size_t)p.NW * 8;
}

// Nibble pair q of a code dword as exact fp16 subnormals: q = 0 -> codes
// e = 0, 1 as u * 2^-24; q = 1 -> e = 2, 3 as 16 u * 2^-24 (nibbles at
// mantissa bits 4-7); q = 2, 3 likewise for e = 4..7 after a shift by 8.
// The partner x carries the factor 1/16 at e in {2, 3, 6, 7}.
__device__ __forceinline__ f16x2_t code_pair_sub(uint32_t w, uint32_t t, int q) {
  const uint32_t v = (q == 0) ? (w & 0x000F000Fu) : (q == 1) ? (w & 0x00F000F0u)
                   : (q == 2) ? (t & 0x000F000Fu) : (t & 0x00F000F0u);
  return bitcast<f16x2_t>(v);
}

// dot of one atom row quarter (4 code dwords) with its 32 x values (fp16
// pairs in k order), times 2^-24
__device__ __forceinline__ float atom_dot(const u32x4_t w, const u32x4_t (&xk)[4]) {
  float acc = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const uint32_t dw = w[kb], t = dw >> 8;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      acc = __builtin_amdgcn_fdot2(code_pair_sub(dw, t, q), bitcast<f16x2_t>(xk[kb][q]), acc, false);
  }
  return acc;
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
// x is staged once per workgroup as fp16 scaled by a power of two sigma
// (max |x| sigma in [2^12, 2^13), so the conversion from bf16 is exact for
// every value above 2^-23 of the row maximum) and by 1/16 at the positions
// paired with the high nibble of a byte.  With GPW > 0 (compile time, a
// divisor of U) each wave keeps its GPW groups of x in registers; GPW == 0
// reads x from LDS for every atom.
template <int EPI, int NW, int U, int GPW>
__global__ __launch_bounds__(NW * 64) void proj_gemv_kernel(ProjArgs a, GemvPlan pl) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int K = a.K, G = a.G;
  const int SP = pl.SP;
  const int GW = GPW > 0 ? GPW : pl.GPW;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                  // [K] fp16
  float* Xs = reinterpret_cast<float*>(smem + (size_t)K * 2);        // [G][4]
  float* red = Xs + (size_t)G * 4;                                   // [SP][NW][16]
  float* ot = red + (size_t)SP * NW * 16;                            // [SP*16]
  float* ssq = ot + SP * 16;                                         // [NW]
  float* wmx = ssq + NW;                                             // [NW]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int r = lane & 15, j = lane >> 4;
  const int nstrips = a.Np / kStrip;
  const int strip0 = blockIdx.x * SP;
  const int ns = min(SP, nstrips - strip0);  // strips of this workgroup
  const int g0 = wave * GW;                   // first group of this wave
  const int gpw = max(0, min(GW, G - g0));    // groups of this wave
  const int n = ns * gpw;                     // atoms of this wave
  const int npad = ((max(n, 1) + U - 1) / U) * U;

  // 1. x: issue the loads of this thread's 16-byte chunks first (clamped,
  // so every thread issues the same number of loads)
  constexpr int XMAX = 4;  // K <= XMAX * 8 * NW * 64 (host-checked)
  u32x4_t xv[XMAX];
#pragma unroll
  for (int q = 0; q < XMAX; ++q) {
    const int cidx = min(tid + q * NW * 64, K / 8 - 1);
    xv[q] = load16(a.x + (size_t)cidx * 8);
  }

  // every wave's x loads enter the memory pipeline before any weight load
  // (otherwise the x of the last waves queues behind the first waves' atoms)
  lds_barrier();

  // 2. the first U atoms of the weight stream.  The refill cursor (rs, rg)
  // walks strip by strip through the wave's groups and stops on the last
  // atom, which pads the sequence.
  int rs = 0, rg = 0;
  auto next_atom = [&](const uint8_t*& cp, const uint16_t*& sp) {
    const int t = min(strip0 + rs, nstrips - 1);
    const int g = min(g0 + rg, G - 1);
    cp = a.codes + ((size_t)t * G + g) * kAtomBytes + (size_t)lane * 16;
    sp = a.scales + (((size_t)t * a.G8 + g / 8) * 16 + r) * 8 + (g % 8);
    if (rs < ns - 1 || rg < gpw - 1) {
      if (++rg >= gpw) {
        rg = 0;
        ++rs;
      }
    }
  };
  u32x4_t ring[U];
  uint16_t sring[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const uint8_t* cp;
    const uint16_t* sp;
    next_atom(cp, sp);
    ring[k] = load16_stream(cp);
    sring[k] = *sp;
  }

  // 3. row statistics: sum of squares (rho) and max |x| (the fp16 scale)
  float sq = 0.f, mx = 0.f;
#pragma unroll
  for (int q = 0; q < XMAX; ++q) {
    if (tid + q * NW * 64 < K / 8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_lo(xv[q][e]), hi = bf16_hi(xv[q][e]);
        sq = fmaf(lo, lo, sq);
        sq = fmaf(hi, hi, sq);
        mx = fmaxf(mx, fmaxf(fabsf(lo), fabsf(hi)));
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    sq += shfl_xor(sq, o);
    mx = fmaxf(mx, shfl_xor(mx, o));
  }
  if (lane == 0) {
    ssq[wave] = sq;
    wmx[wave] = mx;
  }
  lds_barrier();
  float xm = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) xm = fmaxf(xm, wmx[w]);
  int ex = 0;
  if (xm > 0.f) frexpf(xm, &ex);
  const int sh = max(-100, min(100, 13 - ex));
  const float sigma = ldexpf(1.0f, sh);

  // 4. stage x as fp16 (x sigma, / 16 at e in {2,3,6,7})
#pragma unroll
  for (int q = 0; q < XMAX; ++q) {
    const int cidx = tid + q * NW * 64;
    if (cidx < K / 8) {
      u32x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f = (e & 1) ? sigma * 0.0625f : sigma;
        const f16x2_t h = {(_Float16)(bf16_lo(xv[q][e]) * f), (_Float16)(bf16_hi(xv[q][e]) * f)};
        o[e] = bitcast<uint32_t>(h);
      }
      reinterpret_cast<u32x4_t*>(xs)[cidx] = o;
    }
  }
  lds_barrier();

  // 5. x of the wave's groups (registers) or group sums for every group (LDS)
  const u32x4_t* xl = reinterpret_cast<const u32x4_t*>(xs);
  constexpr int GR = GPW > 0 ? GPW : 1;
  u32x4_t xr[GR][4];
  float xsum[GR];
  if (GPW > 0) {
#pragma unroll
    for (int gi = 0; gi < GR; ++gi) {
      const int g = min(g0 + gi, G - 1);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) xr[gi][kb] = xl[(128 * g + 32 * kb + 8 * j) / 8];
      xsum[gi] = quarter_sum(xr[gi]);
    }
  } else {
    for (int idx = tid; idx < G * 4; idx += NW * 64) {
      const int g = idx >> 2, jj = idx & 3;
      u32x4_t xk[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) xk[kb] = xl[(128 * g + 32 * kb + 8 * jj) / 8];
      Xs[idx] = quarter_sum(xk);
    }
    lds_barrier();
  }

  // 6. stream: consume atom i from the ring, then refill its slot with atom
  // i + U (the loaded registers stay in place across iterations)
  float part = 0.f;
  int sl = 0, gi_rt = 0;  // strip and group of the atom being consumed (GPW == 0)
  auto consume = [&](const u32x4_t w, const uint16_t sbits, int i, int k) {
    if (i < n) {
      float y;
      if (GPW > 0) {
        const int gi = k % GR;
        y = fmaf(atom_dot(w, xr[gi]), 16777216.0f, -8.0f * xsum[gi]);
      } else {
        const int g = g0 + gi_rt;
        u32x4_t xk[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) xk[kb] = xl[(128 * g + 32 * kb + 8 * j) / 8];
        y = fmaf(atom_dot(w, xk), 16777216.0f, -8.0f * Xs[g * 4 + j]);
      }
      part = fmaf(f16_bits_to_f32(sbits), y, part);
      const bool last_of_strip = (GPW > 0) ? (k % GR == GR - 1) : (gi_rt == gpw - 1);
      if (last_of_strip) {
        part += shfl_xor(part, 16);
        part += shfl_xor(part, 32);
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
      const uint8_t* cp;
      const uint16_t* sp;
      next_atom(cp, sp);
      ring[k] = load16_stream(cp);
      sring[k] = *sp;
    }
  }
#pragma unroll
  for (int k = 0; k < U; ++k) consume(ring[k], sring[k], i0 + k, k);
  // waves without a group range leave zero partials
  if (j == 0)
    for (int s2 = sl; s2 < ns; ++s2) red[((size_t)s2 * NW + wave) * 16 + r] = 0.f;
  lds_barrier();

  // 7. reduce over the waves and the four lane quarters; undo sigma; epilogue
  if (tid < ns * 16) {
    const int s2 = tid >> 4, rr = tid & 15;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[((size_t)s2 * NW + w) * 16 + rr];
    ot[tid] = v * ldexpf(1.0f, -sh);
  }
  if (needs_rho<EPI>() && tid == 0) {
    float t = 0.f;
    for (int w = 0; w < NW; ++w) t += ssq[w];
    ssq[0] = 1.0f / sqrtf(t / (float)K + a.eps);
  }
  lds_barrier();
  float one = 1.0f;
  run_epilogue<EPI>(a, strip0, ns, ot, needs_rho<EPI>() ? &ssq[0] : &one);
}

// ---------------------------------------------------------------------------
// M = 2..32: bf16 MFMA skinny GEMM
// ---------------------------------------------------------------------------

template <int EPI, int S, int NW, int T>
__global__ __launch_bounds__(NW * 64) void proj_mfma_kernel(ProjArgs a) {
  __shared__ float red[NW][S * 16][T * 16];
  __shared__ float sqred[NW][T * 16];
  __shared__ float rho_s[T * 16];
  __shared__ float ot[S * 16 * T * 16];

  const int K = a.K, G = a.G, M = a.M;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, j = lane >> 4;
  const int strip0 = blockIdx.x * S;
  const int nstrips = a.Np / kStrip;

  const u32x4_t ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const bf16x8_t ones = bitcast<bf16x8_t>(ones_u);

  f32x4_t acc[S][T];
  f32x4_t gram[T];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[s][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < T; ++t) gram[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint8_t* codes = a.codes + (size_t)lane * 16;
  for (int g = wave; g < G; g += NW) {
    u32x4_t w[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int t = strip0 + s;
      w[s] = (t < nstrips) ? load16_stream(codes + ((size_t)t * G + g) * kAtomBytes)
                           : u32x4_t{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
    }
    u32x4_t bx[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int m = 16 * t + r;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        bx[t][kb] = (m < M) ? load16(a.x + (size_t)m * K + 128 * g + 32 * kb + 8 * j)
                            : u32x4_t{0u, 0u, 0u, 0u};
    }
    f32x4_t X[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      X[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8_t b = bitcast<bf16x8_t>(bx[t][kb]);
        X[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, b, X[t], 0, 0, 0);
        if (needs_rho<EPI>()) gram[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, b, gram[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int ts = min(strip0 + s, nstrips - 1);
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc[i] = f16_bits_to_f32(a.scales[(((size_t)ts * a.G8 + g / 8) * 16 + 4 * j + i) * 8 + (g % 8)]);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        f32x4_t ag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dword_to_bf16x8_biased(w[s][kb]),
                                                        bitcast<bf16x8_t>(bx[t][kb]), ag, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[s][t][i] = fmaf(sc[i], ag[i] - 136.0f * X[t][i], acc[s][t][i]);
      }
    }
  }

  // per-wave partials to LDS: lane holds rows 4j+i, column r of each tile
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][s * 16 + 4 * j + i][t * 16 + r] = acc[s][t][i];
  if (needs_rho<EPI>()) {
    // diagonal of x.x^T: element (r, r) sits in lane j = r/4, register r%4
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * j + i == r) sqred[wave][t * 16 + r] = gram[t][i];
  }
  __syncthreads();
  for (int idx = tid; idx < S * 16 * M; idx += NW * 64) {
    const int row = idx / M, m = idx % M;
    float v = 0.f;
    for (int w = 0; w < NW; ++w) v += red[w][row][m];
    ot[row * M + m] = v;
  }
  if (tid < M) {
    float v = 0.f;
    if (needs_rho<EPI>())
      for (int w = 0; w < NW; ++w) v += sqred[w][tid];
    rho_s[tid] = needs_rho<EPI>() ? 1.0f / sqrtf(v / (float)K + a.eps) : 1.0f;
  }
  __syncthreads();
  run_epilogue<EPI>(a, strip0, S, ot, rho_s);
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------

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

template <int EPI, int NW>
static void launch_gemv(const ProjArgs& a, const GemvPlan& p, size_t lds, int grid, hipStream_t st) {
  if (p.GPW == 1)
    hipLaunchKernelGGL((proj_gemv_kernel<EPI, NW, 8, 1>), dim3(grid), dim3(NW * 64), lds, st, a, p);
  else if (p.GPW == 2)
    hipLaunchKernelGGL((proj_gemv_kernel<EPI, NW, 8, 2>), dim3(grid), dim3(NW * 64), lds, st, a, p);
  else if (p.GPW == 4)
    hipLaunchKernelGGL((proj_gemv_kernel<EPI, NW, 4, 4>), dim3(grid), dim3(NW * 64), lds, st, a, p);
  else
    hipLaunchKernelGGL((proj_gemv_kernel<EPI, NW, 8, 0>), dim3(grid), dim3(NW * 64), lds, st, a, p);
}

template <int EPI>
static hipError_t launch_epi(const ProjArgs& a, hipStream_t st) {
  const int nstrips = a.Np / kStrip;
  if (a.M == 1) {
    const GemvPlan p = gemv_plan(nstrips, a.G);
    const size_t lds = gemv_lds_bytes(a.K, p);
    const int grid = (nstrips + p.SP - 1) / p.SP;
    if (p.NW == 16)
      launch_gemv<EPI, 16>(a, p, lds, grid, st);
    else if (p.NW == 8)
      launch_gemv<EPI, 8>(a, p, lds, grid, st);
    else
      launch_gemv<EPI, 4>(a, p, lds, grid, st);
  } else if (a.M <= 16) {
    constexpr int S = 2, NW = 4;
    const int grid = (nstrips + S - 1) / S;
    hipLaunchKernelGGL((proj_mfma_kernel<EPI, S, NW, 1>), dim3(grid), dim3(NW * 64), 0, st, a);
  } else {
    constexpr int S = 2, NW = 4;
    const int grid = (nstrips + S - 1) / S;
    hipLaunchKernelGGL((proj_mfma_kernel<EPI, S, NW, 2>), dim3(grid), dim3(NW * 64), 0, st, a);
  }
  return hipGetLastError();
}

i4d_status launch_projection(int epi, const ProjArgs& a, hipStream_t st) {
  if (a.M == 1) {
    const GemvPlan p = gemv_plan(a.Np / kStrip, a.G);
    const size_t lds = gemv_lds_bytes(a.K, p);
    if (lds > (size_t)kMaxLdsBytes || a.K > 4 * 8 * p.NW * 64)
      return fail(I4D_ERR_UNSUPPORTED, "K=%d too large for the M=1 kernel (LDS %zu bytes)", a.K, lds);
  }
  hipError_t e;
  switch (epi) {
    case EPI_QKV: e = launch_epi<EPI_QKV>(a, st); break;
    case EPI_O: e = launch_epi<EPI_O>(a, st); break;
    case EPI_GU: e = launch_epi<EPI_GU>(a, st); break;
    case EPI_DOWN: e = launch_epi<EPI_DOWN>(a, st); break;
    default: return fail(I4D_ERR_RANGE, "bad epilogue %d", epi);
  }
  if (e != hipSuccess) return fail(I4D_ERR_HIP, "projection launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace i4d
