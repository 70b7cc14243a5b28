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
#include "gemv.h"
#include "i4d_internal.h"
#include "proj.h"

namespace i4d {

constexpr int kMaxLdsBytes = 160 * 1024;

// ---------------------------------------------------------------------------
// M = 1: stand-alone VALU GEMV kernel
// ---------------------------------------------------------------------------

template <int EPI, int NW, int U, int GPW>
__global__ __launch_bounds__(NW * 64) void proj_gemv_kernel(ProjArgs a, GemvPlan pl) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nstrips = a.Np / kStrip;
  const int strip0 = blockIdx.x * pl.SP;
  gemv_body<EPI, NW, U, GPW, false>(a, pl, strip0, min(pl.SP, nstrips - strip0), smem, NoWait());
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
