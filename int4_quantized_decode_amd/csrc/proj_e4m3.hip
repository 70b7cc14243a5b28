// proj_e4m3.hip - projections with E4M3 (FP8) decode weights (gfx950), the
// FP8 decode-weight variant the summary page reports beside the INT4 path
// ("premises and limits"): QKV, O, gate/up, down for M = 1..32 rows.
//
// y[m][n] = sum_g s[n][g] * sum_{k in g} e4m3(c[n][k]) * x[m][k]
//
// The codes are decoded by the hardware conversion to bf16 (every E4M3 value
// is a bf16 value, so the decode is exact) into the A operand of the bf16
// MFMA 16x16x32 (operand row = output row of the atom's strip); T tiles of
// 16 x rows are the B operand, loaded straight from global memory in operand
// order (x is small and shared by every workgroup, so these are L2 hits);
// the group scale is applied after each 128-wide group, as for INT4.
//
// A workgroup of 8 waves owns SP strips; wave w takes groups w, w + 8, ...
// of K, with the next group's atoms, scales and x in flight while it
// computes the current one.  The waves' partial tiles are summed in LDS in
// a fixed order, then the INT4 path's epilogues run (rho, RoPE, residuals,
// SwiGLU).
#include <math.h>

#include "device_common.h"
#include "gemv.h"
#include "i4d_internal.h"
#include "proj.h"

namespace i4d {

constexpr int kE4M3Waves = 8;

// LDS: sums of squares [NW][T*16] | rho [T*16] | tile [SP*16][M] | partial
// tiles [4][SP*16][T*16+4]
inline size_t e4m3_lds_bytes(int SP, int T) {
  return ((size_t)kE4M3Waves * T * 16 + T * 16 + (size_t)SP * 16 * T * 16 + (size_t)4 * SP * 16 * (T * 16 + 4)) * 4;
}

// two E4M3 codes (the low or the high 16 bits of w) -> bf16x2
template <bool HIGH>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH));
}

template <int EPI, int SP, int T>
__global__ __launch_bounds__(kE4M3Waves * 64) void proj_e4m3_kernel(ProjArgs a) {
  constexpr int NW = kE4M3Waves;
  constexpr int RS = T * 16 + 4;
  extern __shared__ __align__(16) unsigned char smem[];
  float* sqw = reinterpret_cast<float*>(smem);  // [NW][T*16]
  float* rho_s = sqw + NW * T * 16;             // [T*16]
  float* ot = rho_s + T * 16;                   // [SP*16][M]
  float* red = ot + SP * 16 * T * 16;           // [4][SP*16][RS]

  const int K = a.K, G = a.G, M = a.M;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int nstrips = a.Np / kStrip;
  const int strip0 = blockIdx.x * SP;
  const int ns = min(SP, nstrips - strip0);
  const int ngw = (G - wave + NW - 1) / NW;  // groups of this wave (0 when G < NW)
  const int nsteps = max(ngw, 1);

  struct Buf {
    u32x4_t w[SP][2];  // the lane's 32 code bytes of each strip's atom
    u32x2_t sc[SP];    // scales of rows 4j .. 4j+3
    u32x4_t x[T][4];   // B operands: row 16t + r, k = 32kb + 8j .. +7 of the group
  };
  // step i of the wave: group wave + NW i (steps past the wave's groups, and
  // a wave without groups, re-read a valid group and weigh it by zero)
  auto load = [&](Buf& b, int i) {
    const int g = min(wave + NW * min(i, nsteps - 1), G - 1);
#pragma unroll
    for (int s = 0; s < SP; ++s) {
      const size_t atom = (size_t)(strip0 + min(s, ns - 1)) * G + g;
      const uint8_t* cp = a.codes + atom * kAtomBytesE4M3 + (size_t)lane * 32;
      b.w[s][0] = load16_stream(cp);
      b.w[s][1] = load16_stream(cp + 16);
      b.sc[s] = *reinterpret_cast<const u32x2_t*>(a.scales + atom * kStrip + 4 * j);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int m = min(16 * t + r, M - 1);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) b.x[t][kb] = load16(a.x + (size_t)m * K + 128 * g + 32 * kb + 8 * j);
    }
  };

  f32x4_t acc[SP][T];
#pragma unroll
  for (int s = 0; s < SP; ++s)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[s][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float sq[T];
#pragma unroll
  for (int t = 0; t < T; ++t) sq[t] = 0.f;

  auto compute = [&](const Buf& b, const bool valid) {
    if (needs_rho<EPI>()) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float q = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            q = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(b.x[t][kb][e]), bitcast<bf16x2_t>(b.x[t][kb][e]), q,
                                                false);
        sq[t] += valid ? q : 0.f;
      }
    }
#pragma unroll
    for (int s = 0; s < SP; ++s) {
      bf16x8_t A[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint32_t d0 = b.w[s][kb >> 1][2 * (kb & 1)], d1 = b.w[s][kb >> 1][2 * (kb & 1) + 1];
        const u32x4_t v = {e4m3x2_to_bf16x2<false>(d0), e4m3x2_to_bf16x2<true>(d0), e4m3x2_to_bf16x2<false>(d1),
                           e4m3x2_to_bf16x2<true>(d1)};
        A[kb] = bitcast<bf16x8_t>(v);
      }
      float scl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sv = f16_bits_to_f32((uint16_t)(b.sc[s][i >> 1] >> (16 * (i & 1))));
        scl[i] = valid ? sv : 0.f;
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        f32x4_t ag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[kb], bitcast<bf16x8_t>(b.x[t][kb]), ag, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[s][t][i] = fmaf(scl[i], ag[i], acc[s][t][i]);
      }
    }
  };

  // two buffers: the next step's loads are in flight while a step computes
  Buf b0, b1;
  load(b0, 0);
  for (int i = 0;; i += 2) {
    if (i + 1 >= nsteps) {
      compute(b0, i < ngw);
      break;
    }
    load(b1, i + 1);
    compute(b0, i < ngw);
    if (i + 2 >= nsteps) {
      compute(b1, i + 1 < ngw);
      break;
    }
    load(b0, i + 2);
    compute(b1, i + 1 < ngw);
  }

  // partial tiles (lane: rows 4j + i of column r of each tile): waves 0-3
  // store, waves 4-7 add theirs to the same slots
  auto slot = [&](int s, int t, int i) { return (((wave & 3) * SP + s) * 16 + 4 * j + i) * RS + t * 16 + r; };
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
  for (int idx = tid; idx < ns * 16 * M; idx += NW * 64) {
    const int row = idx / M, m = idx % M;
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) v += red[((q * SP) * 16 + row) * RS + m];
    ot[idx] = v;
  }
  if (tid < M) {
    float v = 0.f;
    if (needs_rho<EPI>())
      for (int w = 0; w < NW; ++w) v += sqw[w * T * 16 + tid];
    rho_s[tid] = needs_rho<EPI>() ? 1.0f / sqrtf(v / (float)K + a.eps) : 1.0f;
  }
  __syncthreads();
  run_epilogue<EPI>(a, strip0, ns, ot, rho_s);
}

// ---------------------------------------------------------------------------

namespace {

struct E4M3Plan {
  int SP, T, grid;
  size_t lds;
};

// one 16-row x tile up to M = 16, two above; strips per workgroup: the most
// that still gives at least one workgroup per CU (256), at most 4 (one x
// tile) or 2 (two tiles: the register file)
E4M3Plan e4m3_plan(int nstrips, int M) {
  E4M3Plan p;
  p.T = M <= 16 ? 1 : 2;
  p.SP = 1;
  for (int sp : {4, 2}) {
    if ((p.T == 2 && sp > 2) || (nstrips + sp - 1) / sp < 256) continue;
    p.SP = sp;
    break;
  }
  p.grid = (nstrips + p.SP - 1) / p.SP;
  p.lds = e4m3_lds_bytes(p.SP, p.T);
  return p;
}

template <int EPI>
bool launch_e4m3_epi(const ProjArgs& a, const E4M3Plan& p, hipStream_t st) {
#define I4D_E4M3(SPV, TV)                                                                                   \
  if (p.SP == SPV && p.T == TV) {                                                                           \
    hipLaunchKernelGGL((proj_e4m3_kernel<EPI, SPV, TV>), dim3(p.grid), dim3(kE4M3Waves * 64), p.lds, st, a); \
    return true;                                                                                            \
  }
  I4D_E4M3(1, 1) I4D_E4M3(2, 1) I4D_E4M3(4, 1) I4D_E4M3(1, 2) I4D_E4M3(2, 2)
#undef I4D_E4M3
  return false;
}

}  // namespace

i4d_status launch_projection_e4m3(int epi, const ProjArgs& a, hipStream_t st) {
  if (a.M < 1 || a.M > I4D_MAX_ROWS) return fail(I4D_ERR_RANGE, "M=%d outside [1, 32]", a.M);
  const E4M3Plan p = e4m3_plan(a.Np / kStrip, a.M);
  bool launched;
  switch (epi) {
    case EPI_QKV: launched = launch_e4m3_epi<EPI_QKV>(a, p, st); break;
    case EPI_O: launched = launch_e4m3_epi<EPI_O>(a, p, st); break;
    case EPI_GU: launched = launch_e4m3_epi<EPI_GU>(a, p, st); break;
    case EPI_DOWN: launched = launch_e4m3_epi<EPI_DOWN>(a, p, st); break;
    default: return fail(I4D_ERR_RANGE, "bad epilogue %d", epi);
  }
  if (!launched) return fail(I4D_ERR_UNSUPPORTED, "no E4M3 projection kernel for SP %d, T %d", p.SP, p.T);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(I4D_ERR_HIP, "E4M3 projection launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace i4d
