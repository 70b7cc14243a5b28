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

constexpr int kMaxLdsBytes = 65536;

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
template <int EPI, int S>
__device__ void run_epilogue(const ProjArgs& a, int strip0, const float* ot, const float* rho) {
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

template <int U, int S, bool NT>
__device__ __forceinline__ void gemv_issue(u32x4_t (&w)[U][S], const uint8_t* codes, int strip0,
                                           int nstrips, int G, int g0, int NW) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int g = g0 + u * NW;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int t = strip0 + s;
      if (g < G && t < nstrips)
        w[u][s] = NT ? load16_stream(codes + ((size_t)t * G + g) * kAtomBytes)
                     : load16(codes + ((size_t)t * G + g) * kAtomBytes);
      else
        w[u][s] = u32x4_t{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
    }
  }
}

template <int EPI, int S, int NW, int U, bool NT>
__global__ __launch_bounds__(NW * 64) void proj_gemv_kernel(ProjArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int K = a.K, G = a.G;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                 // [K] bf16
  float* Xs = reinterpret_cast<float*>(smem + (size_t)K * 2);       // [G][4] chunk sums
  float* red = Xs + (size_t)G * 4;                                  // [NW][S*16]
  float* ot = red + NW * S * 16;                                    // [S*16]
  float* misc = ot + S * 16;                                        // [NW] + rho

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, j = lane >> 4;
  const int strip0 = blockIdx.x * S;
  const int nstrips = a.Np / kStrip;
  const uint8_t* codes = a.codes + (size_t)lane * 16;

  // the weight stream does not depend on x: start it before staging x
  // (U groups per batch and wave, two batches in flight)
  u32x4_t wa[U][S], wb[U][S];
  gemv_issue<U, S, NT>(wa, codes, strip0, nstrips, G, wave, NW);

  // stage x (bf16) in LDS and accumulate its sum of squares
  float sq = 0.f;
  {
    const u32x4_t* xg = reinterpret_cast<const u32x4_t*>(a.x);
    u32x4_t* xl = reinterpret_cast<u32x4_t*>(xs);
    for (int c = tid; c < K / 8; c += NW * 64) {
      const u32x4_t v = xg[c];
      xl[c] = v;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = bf16_lo(v[q]), hi = bf16_hi(v[q]);
        sq = fmaf(lo, lo, sq);
        sq = fmaf(hi, hi, sq);
      }
    }
  }
  if (needs_rho<EPI>()) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sq += shfl_xor(sq, o);
    if (lane == 0) misc[wave] = sq;
  }
  __syncthreads();
  // group sums over the 32 codes each lane (j) of a group multiplies
  for (int idx = tid; idx < G * 4; idx += NW * 64) {
    const int g = idx >> 2, jj = idx & 3;
    const u32x4_t* xl = reinterpret_cast<const u32x4_t*>(xs);
    float sm = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const u32x4_t v = xl[(128 * g + 32 * kb + 8 * jj) / 8];
#pragma unroll
      for (int q = 0; q < 4; ++q) sm += bf16_lo(v[q]) + bf16_hi(v[q]);
    }
    Xs[idx] = sm;
  }
  if (needs_rho<EPI>() && tid == 0) {
    float t = 0.f;
    for (int w = 0; w < NW; ++w) t += misc[w];
    misc[NW] = 1.0f / sqrtf(t / (float)K + a.eps);
  }
  __syncthreads();

  float part[S];
#pragma unroll
  for (int s = 0; s < S; ++s) part[s] = 0.f;

  const u32x4_t* xl = reinterpret_cast<const u32x4_t*>(xs);
  auto consume = [&](u32x4_t (&w)[U][S], int g0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = g0 + u * NW;
      if (g >= G) break;
      u32x4_t xv[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) xv[kb] = xl[(128 * g + 32 * kb + 8 * j) / 8];
      const float corr = 136.0f * Xs[g * 4 + j];
#pragma unroll
      for (int s = 0; s < S; ++s) {
        float acc = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const uint32_t dw = w[u][s][kb];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(nib_pair_bf16(dw, i)),
                                                  bitcast<bf16x2_t>(xv[kb][i]), acc, false);
        }
        const int t = min(strip0 + s, nstrips - 1);
        const float sc = f16_bits_to_f32(a.scales[(((size_t)t * a.G8 + g / 8) * 16 + r) * 8 + (g % 8)]);
        part[s] = fmaf(sc, acc - corr, part[s]);
      }
    }
  };
  // double-buffered batches of U groups: issue batch b+1, then consume batch b
  for (int g0 = wave;; g0 += 2 * NW * U) {
    const int g1 = g0 + NW * U;
    if (g1 < G) gemv_issue<U, S, NT>(wb, codes, strip0, nstrips, G, g1, NW);
    consume(wa, g0);
    if (g1 >= G) break;
    const int g2 = g1 + NW * U;
    if (g2 < G) gemv_issue<U, S, NT>(wa, codes, strip0, nstrips, G, g2, NW);
    consume(wb, g1);
    if (g2 >= G) break;
  }
#pragma unroll
  for (int s = 0; s < S; ++s) {
    part[s] += shfl_xor(part[s], 16);
    part[s] += shfl_xor(part[s], 32);
  }
  if (j == 0) {
#pragma unroll
    for (int s = 0; s < S; ++s) red[wave * S * 16 + s * 16 + r] = part[s];
  }
  __syncthreads();
  if (tid < S * 16) {
    float v = 0.f;
    for (int w = 0; w < NW; ++w) v += red[w * S * 16 + tid];
    ot[tid] = v;
  }
  __syncthreads();
  float one = 1.0f;
  run_epilogue<EPI, S>(a, strip0, ot, needs_rho<EPI>() ? &misc[NW] : &one);
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
  run_epilogue<EPI, S>(a, strip0, ot, rho_s);
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------

// waves per workgroup of the M = 1 kernel: enough waves in flight (>= 2048)
// and at most 8 groups per wave when the shape allows
static int gemv_waves(int nstrips, int G) {
  int nw = 4;
  while (nw < 16 && ((long)nstrips * nw < 2048 || (G + nw - 1) / nw > 8)) nw *= 2;
  while (nw > 4 && nw > G) nw /= 2;
  return nw;
}

template <int EPI>
static hipError_t launch_epi(const ProjArgs& a, hipStream_t st) {
  const int nstrips = a.Np / kStrip;
  if (a.M == 1) {
    constexpr int S = 1;
    const int nw = gemv_waves(nstrips, a.G);
    const size_t lds = gemv_lds_bytes(a.K, S, nw);
    const int grid = (nstrips + S - 1) / S;
    if (nw == 4)
      hipLaunchKernelGGL((proj_gemv_kernel<EPI, S, 4, 8, true>), dim3(grid), dim3(4 * 64), lds, st, a);
    else if (nw == 8)
      hipLaunchKernelGGL((proj_gemv_kernel<EPI, S, 8, 8, true>), dim3(grid), dim3(8 * 64), lds, st, a);
    else
      hipLaunchKernelGGL((proj_gemv_kernel<EPI, S, 16, 8, true>), dim3(grid), dim3(16 * 64), lds, st, a);
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
    const size_t lds = gemv_lds_bytes(a.K, 1, 16);
    if (lds > (size_t)kMaxLdsBytes)
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
