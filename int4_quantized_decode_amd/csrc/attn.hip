// attn.hip - INT4 KV cache append and GQA split-KV flash-decode (gfx950).
//
// kv_append: one wave per (token, kv head, K|V).  The head_dim values are
//   spread over the 64 lanes, rotated by the unnormalised fast Walsh-Hadamard
//   transform in fp32 (stage order h = 1, 2, 4, ...; cross-lane stages use
//   lane shuffles, the add DAG is the same as the plain transform so the
//   result is bit-identical), reduced to the absmax, quantized with
//   scale = fp16(absmax / 7) (correctly rounded fp32 division) and written in
//   the MFMA operand layout of the cache ("how it differs": rotation before
//   cache quantization; "how it works": direct placement at
//   offset(request, head, position, channel)).
//
// attention: one workgroup per (row, kv head, split); its waves take
//   interleaved 32-token blocks.  Per block:
//     S[token][col]  = K_codes(16 tokens x hd, fp16) . [q~_hi | q~_lo]  (MFMA)
//     online softmax in fp32 (log2 domain), p' = p * v_scale
//     O[ch][col]    += V_codes^T(16 ch x 32 tokens, fp16) . [p'_hi | p'_lo]
//   The G query heads of the kv head share every K/V load ("premises and
//   limits": the 8-head cache is read without expanding it).  Columns 0..G-1
//   carry the high fp16 part of q~ / p', columns G..2G-1 the low part, so
//   scores and outputs keep ~fp32 precision on fp16 MFMA.  The waves merge in
//   LDS and write one (max, sum, output) partial per split; the combine
//   kernel merges the splits and applies the inverse rotation H o~ / hd
//   ("how it differs": split-KV reduction, same rotation on the output).
#include <math.h>

#include "attn.h"
#include "device_common.h"

namespace i4d {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ uint16_t f32_to_f16_sat(float f) {
  _Float16 h = (_Float16)f;  // round to nearest even
  uint16_t b = bitcast<uint16_t>(h);
  if ((b & 0x7fffu) == 0x7c00u && isfinite(f)) b = (uint16_t)((b & 0x8000u) | 0x7bffu);
  return b;
}

// ---------------------------------------------------------------------------
// append
// ---------------------------------------------------------------------------

template <int HD>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * 4 + (threadIdx.x >> 6);
  const KvArgs& kv = a.kv;
  if (idx >= a.T * kv.n_kv * 2) return;
  const int kind = idx & 1;
  const int rest = idx >> 1;
  const int head = rest % kv.n_kv;
  const int t = rest / kv.n_kv;
  const int row = a.row_idx ? a.row_idx[t] : t;
  const int pos = a.len ? a.len[t] - 1 : a.pos[t];
  if (row < 0 || row >= kv.n_rows) {
    if (lane == 0 && kv.err_word) atomicOr(kv.err_word, I4D_DEVERR_APPEND_POS);
    return;
  }
  const int64_t base = kv.row_base[row];
  const int64_t cap = kv.row_base[row + 1] - base;
  if (pos < 0 || pos >= cap) {
    if (lane == 0 && kv.err_word) atomicOr(kv.err_word, I4D_DEVERR_APPEND_POS);
    return;
  }
  const uint16_t* src = (kind ? a.v : a.k) + ((size_t)t * kv.n_kv + head) * HD;
  float x0 = bf16_to_f32(src[lane]);
  float x1 = (HD == 128) ? bf16_to_f32(src[lane + 64]) : 0.f;
  // FWHT, stages h = 1 .. 32 across lanes, then h = 64 inside the lane
#pragma unroll
  for (int h = 1; h < 64 && h < HD; h <<= 1) {
    const float p0 = shfl_xor(x0, h);
    x0 = (lane & h) ? (p0 - x0) : (x0 + p0);
    if (HD == 128) {
      const float p1 = shfl_xor(x1, h);
      x1 = (lane & h) ? (p1 - x1) : (x1 + p1);
    }
  }
  if (HD == 128) {
    const float s0 = x0 + x1, s1 = x0 - x1;
    x0 = s0;
    x1 = s1;
  }
  const float amax = wave_max(fmaxf(fabsf(x0), (HD == 128) ? fabsf(x1) : 0.f));
  const uint16_t s16 = f32_to_f16_sat(__fdiv_rn(amax, 7.0f));
  const float sf = f16_bits_to_f32(s16);
  int u0 = 8, u1 = 8;
  if (sf != 0.f) {
    u0 = (int)fminf(7.f, fmaxf(-8.f, rintf(__fdiv_rn(x0, sf)))) + 8;
    u1 = (int)fminf(7.f, fmaxf(-8.f, rintf(__fdiv_rn(x1, sf)))) + 8;
  }
  const int64_t region = base * kv.n_kv + (int64_t)head * cap;  // first slot of (row, head)
  const int64_t slot = region + pos;
  if (kind == 0) {
    // key slot: dword d = jj*(HD/32) + kb holds channels 32kb + 8jj + e
    uint32_t word = 0;
    const int d = lane;
    const int jj = d / (HD / 32), kb = d % (HD / 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 32 * kb + 8 * jj + e;
      const int src_lane = c & 63;
      const int v0 = __shfl(u0, src_lane, 64);
      const int v1 = __shfl(u1, src_lane, 64);
      const int u = (c < 64) ? v0 : v1;
      word |= (uint32_t)u << (4 * nibble_slot(e));
    }
    if (d < HD / 8) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(kv.k_codes + (size_t)slot * (HD / 2));
      dst[d] = word;
    }
    if (lane == 0) kv.k_scales[slot] = s16;
  } else {
    const int w = pos % kVBlock;
    int jj, e;
    if (w < 16) {
      jj = w / 4;
      e = w % 4;
    } else {
      jj = (w - 16) / 4;
      e = 4 + (w - 16) % 4;
    }
    const int sh = 4 * nibble_slot(e);
    uint32_t* blk = kv.v_codes + (size_t)(region / kVBlock + pos / kVBlock) * 4 * HD;
#pragma unroll
    for (int q = 0; q < HD / 64; ++q) {
      const int c = lane + 64 * q;
      const int u = q ? u1 : u0;
      uint32_t* dw = blk + jj * HD + (c % 16) * (HD / 16) + c / 16;
      atomicAnd(dw, ~(0xFu << sh));
      atomicOr(dw, (uint32_t)u << sh);
    }
    if (lane == 0) kv.v_scales[slot] = s16;
  }
}

// ---------------------------------------------------------------------------
// split flash-decode
// ---------------------------------------------------------------------------

template <int HD>
__global__ __launch_bounds__(kAttnWaves * 64) void attn_split_kernel(AttnArgs a) {
  constexpr int NWA = kAttnWaves;
  constexpr int KB = HD / 32;  // 32-channel MFMA steps for q.k
  constexpr int CB = HD / 16;  // 16-channel output blocks
  __shared__ float wm[NWA][8];
  __shared__ float wl[NWA][8];
  __shared__ float wo[NWA][8][HD];

  const KvArgs& kv = a.kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, jj = lane >> 4;
  const int S = a.S, G = a.G;
  const int s = blockIdx.x % S;
  const int rest = blockIdx.x / S;
  const int j = rest % kv.n_kv;
  const int m = rest / kv.n_kv;

  const int64_t base = kv.row_base[m];
  const int64_t cap = kv.row_base[m + 1] - base;
  int L = a.ctx_len[m];
  if (L < 1 || L > cap) {
    if (tid == 0 && kv.err_word) atomicOr(kv.err_word, I4D_DEVERR_CTX_LEN);
    L = (int)max((int64_t)0, min((int64_t)max(L, 1), cap));
  }
  const int nblk = (L + kVBlock - 1) / kVBlock;
  const int bps = (nblk + S - 1) / S;
  const int b0 = s * bps;
  const int b1 = min(nblk, b0 + bps);
  const int64_t region = base * kv.n_kv + (int64_t)j * cap;

  // --- rotated query, fp16 hi/lo B operands: column c -> head c % G (c < 2G)
  f16x8_t qhi[KB], qlo[KB];
  {
    float qv[KB][8];
    const bool active = c < 2 * G;
    const int g = c % G;
    const float* qsrc = a.q + ((size_t)m * a.n_q + (size_t)j * G + g) * HD + 8 * jj;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (active) {
        const u32x4_t v0 = load16(qsrc + 32 * kb);
        const u32x4_t v1 = load16(qsrc + 32 * kb + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qv[kb][e] = __uint_as_float(v0[e]);
          qv[kb][4 + e] = __uint_as_float(v1[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[kb][e] = 0.f;
      }
    }
    // channel = 32*kb + 8*jj + e: bits 0-2 in-lane (e), 3-4 across lanes
    // (jj: lane ^ 16, lane ^ 32), 5-6 in-lane (kb)
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (!(e & h)) {
            const float x = qv[kb][e], y = qv[kb][e + h];
            qv[kb][e] = x + y;
            qv[kb][e + h] = x - y;
          }
#pragma unroll
    for (int hl = 16; hl <= 32; hl <<= 1) {
      const bool upper = (lane & hl) != 0;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = shfl_xor(qv[kb][e], hl);
          qv[kb][e] = upper ? (p - qv[kb][e]) : (qv[kb][e] + p);
        }
    }
#pragma unroll
    for (int h = 1; h < KB; h <<= 1)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        if (!(kb & h))
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = qv[kb][e], y = qv[kb + h][e];
            qv[kb][e] = x + y;
            qv[kb + h][e] = x - y;
          }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const _Float16 hi = (_Float16)qv[kb][e];
        qhi[kb][e] = hi;
        qlo[kb][e] = (_Float16)(qv[kb][e] - (float)hi);
      }
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint8_t* kbase = kv.k_codes + (size_t)region * (HD / 2);
  const uint16_t* ksc = kv.k_scales + region;
  const uint16_t* vsc = kv.v_scales + region;
  const uint32_t* vbase = kv.v_codes + (size_t)(region / kVBlock) * 4 * HD;
  const float sscale = a.score_scale;

  for (int blk = b0 + wave; blk < b1; blk += NWA) {
    const int t0 = blk * kVBlock;
    // loads: keys for 2 tiles of 16 tokens (lane row = token c), values,
    // scales for the tokens whose scores this lane holds (t0 + 16 tile + 4 jj + i)
    uint32_t kw[2][KB];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const uint8_t* kp = kbase + (size_t)(t0 + 16 * tile + c) * (HD / 2) + jj * (HD / 8);
      if (HD == 128) {
        const u32x4_t v = load16(kp);
        kw[tile][0] = v.x;
        kw[tile][1] = v.y;
        kw[tile][2] = v.z;
        kw[tile][3] = v.w;
      } else {
        const u32x2_t v = *reinterpret_cast<const u32x2_t*>(kp);
        kw[tile][0] = v.x;
        kw[tile][1] = v.y;
      }
    }
    uint32_t vw[CB];
    {
      const uint32_t* vp = vbase + (size_t)blk * 4 * HD + jj * HD + c * CB;
#pragma unroll
      for (int q = 0; q < CB / 4; ++q) {
        const u32x4_t v = load16(vp + 4 * q);
        vw[4 * q + 0] = v.x;
        vw[4 * q + 1] = v.y;
        vw[4 * q + 2] = v.z;
        vw[4 * q + 3] = v.w;
      }
    }
    u32x2_t ks2[2], vs2[2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      ks2[tile] = *reinterpret_cast<const u32x2_t*>(ksc + t0 + 16 * tile + 4 * jj);
      vs2[tile] = *reinterpret_cast<const u32x2_t*>(vsc + t0 + 16 * tile + 4 * jj);
    }

    // scores
    float sc[8];
    float mx = -INFINITY;
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const f16x8_t kf = dword_to_f16x8_signed(kw[tile][kb]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qhi[kb], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qlo[kb], acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 16 * tile + 4 * jj + i;
        const uint32_t word = ks2[tile][i >> 1];
        const float ks = f16_bits_to_f32((uint16_t)((i & 1) ? (word >> 16) : (word & 0xffffu)));
        const float v = (tok < L) ? acc[i] * ks * sscale : -INFINITY;
        sc[tile * 4 + i] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) o[cb] *= alpha;

    f16x8_t pb;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int tile = q >> 2, i = q & 3;
      const int tok = t0 + 16 * tile + 4 * jj + i;
      const uint32_t word = vs2[tile][i >> 1];
      const float vs = f16_bits_to_f32((uint16_t)((i & 1) ? (word >> 16) : (word & 0xffffu)));
      const float p = (tok < L) ? exp2f(sc[q] - m_new) : 0.f;
      l_run += p;
      const float pv = (tok < L) ? p * vs : 0.f;
      const _Float16 hi = (_Float16)pv;
      const _Float16 lo = (_Float16)(pv - (float)hi);
      pb[q] = (c < G) ? hi : ((c < 2 * G) ? lo : (_Float16)0.0f);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dword_to_f16x8_signed(vw[cb]), pb, o[cb], 0, 0, 0);
    m_run = m_new;
  }

  // merge the four lane rows (jj) of l, and the hi/lo columns of o
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[cb][i] += __shfl_xor(o[cb][i], G, 64);

  if (c < G) {
    if (jj == 0) {
      wm[wave][c] = m_run;
      wl[wave][c] = l_run;
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) wo[wave][c][16 * cb + 4 * jj + i] = o[cb][i];
  }
  __syncthreads();

  // merge the waves and write this split's partial for the G heads
  for (int idx = tid; idx < G * HD; idx += NWA * 64) {
    const int g = idx / HD, ch = idx % HD;
    float M_ = -INFINITY;
    for (int w = 0; w < NWA; ++w)
      if (wl[w][g] > 0.f) M_ = fmaxf(M_, wm[w][g]);
    float lsum = 0.f, osum = 0.f;
    for (int w = 0; w < NWA; ++w) {
      if (wl[w][g] > 0.f) {
        const float f = exp2f(wm[w][g] - M_);
        lsum += f * wl[w][g];
        osum += f * wo[w][g][ch];
      }
    }
    const size_t ph = ((size_t)m * a.n_q + (size_t)j * G + g) * S + s;
    a.part_o[ph * HD + ch] = osum;
    if (ch == 0) {
      a.part_ml[ph * 2] = M_;
      a.part_ml[ph * 2 + 1] = lsum;
    }
  }
}

// combine the splits of one (row, q head) and undo the rotation: o = H o~ / hd
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= a.M * a.n_q) return;
  const int S = a.S;
  const float* ml = a.part_ml + (size_t)idx * S * 2;
  const float* po = a.part_o + (size_t)idx * S * HD;
  float M_ = -INFINITY;
  for (int s = 0; s < S; ++s)
    if (ml[2 * s + 1] > 0.f) M_ = fmaxf(M_, ml[2 * s]);
  float lsum = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < S; ++s) {
    const float l = ml[2 * s + 1];
    if (l > 0.f) {
      const float f = exp2f(ml[2 * s] - M_);
      lsum += f * l;
      o0 += f * po[(size_t)s * HD + lane];
      if (HD == 128) o1 += f * po[(size_t)s * HD + lane + 64];
    }
  }
  const float inv = 1.0f / lsum;
  o0 *= inv;
  o1 *= inv;
#pragma unroll
  for (int h = 1; h < 64 && h < HD; h <<= 1) {
    const float p0 = shfl_xor(o0, h);
    o0 = (lane & h) ? (p0 - o0) : (o0 + p0);
    if (HD == 128) {
      const float p1 = shfl_xor(o1, h);
      o1 = (lane & h) ? (p1 - o1) : (o1 + p1);
    }
  }
  if (HD == 128) {
    const float s0 = o0 + o1, s1 = o0 - o1;
    o0 = s0;
    o1 = s1;
  }
  const float scale = 1.0f / (float)HD;
  o0 *= scale;
  o1 *= scale;
  const size_t base = (size_t)idx * HD;
  if (a.attn_f32) {
    a.attn_f32[base + lane] = o0;
    if (HD == 128) a.attn_f32[base + lane + 64] = o1;
  }
  a.attn_bf16[base + lane] = f32_to_bf16(o0);
  if (HD == 128) a.attn_bf16[base + lane + 64] = f32_to_bf16(o1);
}

// ---------------------------------------------------------------------------

i4d_status launch_kv_append(const AppendArgs& a, hipStream_t st) {
  const int waves = a.T * a.kv.n_kv * 2;
  if (waves == 0) return ok();
  const int grid = (waves + 3) / 4;
  if (a.kv.hd == 128)
    hipLaunchKernelGGL(kv_append_kernel<128>, dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<64>, dim3(grid), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(I4D_ERR_HIP, "kv_append launch: %s", hipGetErrorString(e));
  return ok();
}

i4d_status launch_kv_append_at_len(AppendArgs a, const int32_t* ctx_len, hipStream_t st) {
  a.len = ctx_len;
  a.pos = nullptr;
  a.row_idx = nullptr;
  return launch_kv_append(a, st);
}

i4d_status launch_attention(const AttnArgs& a, hipStream_t st) {
  const int grid = a.M * a.kv.n_kv * a.S;
  const int cgrid = (a.M * a.n_q + 3) / 4;
  if (a.kv.hd == 128) {
    hipLaunchKernelGGL(attn_split_kernel<128>, dim3(grid), dim3(kAttnWaves * 64), 0, st, a);
    hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(cgrid), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(attn_split_kernel<64>, dim3(grid), dim3(kAttnWaves * 64), 0, st, a);
    hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(cgrid), dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(I4D_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace i4d
