// lmhead.hip - final RMSNorm factor + bf16 LM head + greedy argmax (gfx950).
//
// logits[m][v] = rho_f[m] * sum_k h[m][k] w[v][k]; the final-norm gain is
// folded into the bf16 weight on the host.  One wave owns two 16-row vocab
// strips and the full d: the weight rows are the A operand of the bf16 MFMA
// 16x16x32 (lane row = vocab row, 8 consecutive k), h rows are the B
// operand, and h . h^T on the same MFMA gives the
// sum of squares for rho_f.  The weight is stored in tiles of 16 rows x 32
// k, so each 16-byte operand load of a wave reads one contiguous KiB (row
// order read 16 rows x 64 bytes per load: 4.4 against 5.8 TB/s measured at
// 128256 x 4096).  Each wave writes its best (value, index) per row
// m; a second kernel reduces them with ties going to the lowest index.
#include <math.h>

#include "device_common.h"
#include "i4d_internal.h"
#include "lmhead.h"

namespace i4d {

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int T>
__global__ __launch_bounds__(kLmWavesPerBlock * 64) void lm_head_kernel(LmArgs a) {
  constexpr int SW = kLmStripsPerWave;
  const int lane = threadIdx.x & 63, r = lane & 15, j = lane >> 4;
  const int wg = blockIdx.x * kLmWavesPerBlock + (threadIdx.x >> 6);
  if (wg >= a.nwaves) return;
  const int nstrips = a.V / kStrip;
  const int d = a.d, M = a.M;

  f32x4_t acc[SW][T], gram[T];
#pragma unroll
  for (int s = 0; s < SW; ++s)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[s][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < T; ++t) gram[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint16_t* wrow[SW];
  bool svalid[SW];
#pragma unroll
  for (int s = 0; s < SW; ++s) {
    const int st = wg * SW + s;
    svalid[s] = st < nstrips;
    wrow[s] = a.w + (size_t)(svalid[s] ? st : 0) * kStrip * d + r * 32 + 8 * j;  // tile 0 of strip st
  }
  constexpr int U = 4;
  for (int k0 = 0; k0 < d; k0 += 32 * U) {
    u32x4_t wv[U][SW], bx[U][T];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + 32 * u;
#pragma unroll
      for (int s = 0; s < SW; ++s)
        wv[u][s] = (svalid[s] && k < d) ? load16_stream(wrow[s] + (size_t)(k / 32) * (kStrip * 32))
                                        : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int m = 16 * t + r;
        bx[u][t] = (m < M && k < d) ? load16(a.h + (size_t)m * d + k + 8 * j) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const bf16x8_t b = bitcast<bf16x8_t>(bx[u][t]);
        gram[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, b, gram[t], 0, 0, 0);
#pragma unroll
        for (int s = 0; s < SW; ++s)
          acc[s][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(wv[u][s]), b,
                                                              acc[s][t], 0, 0, 0);
      }
  }

#pragma unroll
  for (int t = 0; t < T; ++t) {
    // rho_f for column m = 16t + r: diagonal element (r, r) is held by lane
    // (r/4)*16 + r in register r % 4
    float diag = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * j + i == r) diag = gram[t][i];
    const float sq = __shfl(diag, (r >> 2) * 16 + r, 64);
    const float rho = 1.0f / sqrtf(sq / (float)d + a.eps);
    const int m = 16 * t + r;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int s = 0; s < SW; ++s) {
      if (!svalid[s]) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = (wg * SW + s) * kStrip + 4 * j + i;
        const float val = rho * acc[s][t][i];
        if (a.logits && m < M) a.logits[(size_t)m * a.V + v] = val;
        if (better(val, v, bv, bi)) {
          bv = val;
          bi = v;
        }
      }
    }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float ov = shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (j == 0 && m < M) {
      a.part_val[(size_t)wg * M + m] = bv;
      a.part_idx[(size_t)wg * M + m] = bi;
    }
  }
}

__global__ __launch_bounds__(256) void lm_argmax_final_kernel(LmArgs a) {
  __shared__ float sv[256];
  __shared__ int si[256];
  const int m = blockIdx.x, tid = threadIdx.x;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int w = tid; w < a.nwaves; w += 256) {
    const float v = a.part_val[(size_t)w * a.M + m];
    const int i = a.part_idx[(size_t)w * a.M + m];
    if (better(v, i, bv, bi)) {
      bv = v;
      bi = i;
    }
  }
  sv[tid] = bv;
  si[tid] = bi;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if (tid < o && better(sv[tid + o], si[tid + o], sv[tid], si[tid])) {
      sv[tid] = sv[tid + o];
      si[tid] = si[tid + o];
    }
    __syncthreads();
  }
  if (tid == 0) a.token[m] = (si[0] == 0x7fffffff) ? 0 : si[0];
}

i4d_status launch_lm_head(const LmArgs& a, hipStream_t st) {
  const int grid = (a.nwaves + kLmWavesPerBlock - 1) / kLmWavesPerBlock;
  if (a.M <= 16)
    hipLaunchKernelGGL(lm_head_kernel<1>, dim3(grid), dim3(kLmWavesPerBlock * 64), 0, st, a);
  else
    hipLaunchKernelGGL(lm_head_kernel<2>, dim3(grid), dim3(kLmWavesPerBlock * 64), 0, st, a);
  hipLaunchKernelGGL(lm_argmax_final_kernel, dim3(a.M), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(I4D_ERR_HIP, "lm head launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace i4d
