// attn_core.h - INT4 KV append and GQA decode attention as device functions,
// shared by the stand-alone kernels and the one-launch decode step.
//
// Append: one wave rotates one key or value vector with the unnormalised fast
//   Walsh-Hadamard transform in fp32 (stage order h = 1, 2, 4, ...; the
//   cross-lane stages use lane shuffles with the same add DAG as the plain
//   transform, so the result is bit-identical), takes the absmax, quantizes
//   with scale = fp16(absmax / 7) (correctly rounded fp32 division) and writes
//   the codes in the MFMA operand layout of the cache ("how it differs":
//   rotation before cache quantization; "how it works": direct placement at
//   offset(request, head, position, channel)).
//
// Attention: one workgroup per (row, kv head, split) with 4 or 8 waves
//   that take interleaved 32-token blocks.  Per block and wave:
//     S[token][col] = K_codes(16 tokens x hd) . q~  (MFMA, fp16; the rotated
//                     query's high part in columns c < 8, its residual in
//                     columns 8 + c, recombined by a DPP row rotation)
//     online softmax in fp32 (log2 domain), p' = p * v_scale (fp16)
//     O[ch][col]   += V_codes^T(16 channels x 32 tokens, fp16) . p'  (MFMA)
//   Column c of both products is query head c of the kv head, so the G heads
//   share every K/V load ("premises and limits": the 8-head cache is read
//   without expanding it).  The waves merge in LDS; with one split the
//   workgroup normalises and undoes the rotation (o = H o~ / hd) itself,
//   otherwise it writes (max, sum, output) partials that a combine step
//   merges ("how it differs": split-KV reduction, same rotation on the
//   output).  In a decode step the workgroup whose split holds position L-1
//   first appends the step's new key and value.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "attn.h"
#include "coherent.h"
#include "device_common.h"

namespace i4d {

__device__ __forceinline__ float wave_max(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, lane_xor(v, o, lane));
  return v;
}

__device__ __forceinline__ uint16_t f32_to_f16_sat(float f) {
  _Float16 h = (_Float16)f;  // round to nearest even
  uint16_t b = bitcast<uint16_t>(h);
  if ((b & 0x7fffu) == 0x7c00u && isfinite(f)) b = (uint16_t)((b & 0x8000u) | 0x7bffu);
  return b;
}

// ---------------------------------------------------------------------------
// append of one vector by one wave
// ---------------------------------------------------------------------------

// region = first slot of (row, head); pos < capacity; kind 0 = key, 1 = value.
// With `nt` the codes and the scale are also written to LDS (NewToken).
struct NewToken {
  uint32_t kw[32];  // the key's cache words (HD / 8 of them)
  uint8_t v[128];   // the value's codes, one per channel
  uint16_t ks, vs;  // fp16 scales
};

// poll the flagged words p[lane] and p[lane + 64] (HD = 128) until both hold
// `flag`; their low 32 bits into d0, d1
template <int HD>
__device__ __forceinline__ void poll_pair(const uint64_t* p, int lane, uint32_t flag, unsigned* sync_err,
                                          int32_t* err_word, uint32_t& d0, uint32_t& d1) {
  uint64_t w0 = 0, w1 = 0;
  for (int it = 0;; ++it) {
    // both loads in flight before either is tested (no branch between)
    w0 = ld_flag(&p[lane]);
    w1 = (HD == 128) ? ld_flag(&p[lane + 64]) : ((uint64_t)flag << 32);
    if (__all(flag_is(w0, flag) & flag_is(w1, flag))) break;
    if (it == kPollLimit) {
      poll_timeout(sync_err, err_word);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  d0 = (uint32_t)w0;
  d1 = (uint32_t)w1;
}

// COH (one-launch step): the vector comes from the flagged words src_ll
// [HD] (bf16 bits) instead of src
template <int HD, bool COH = false>
__device__ void append_vector(const KvArgs& kv, const uint16_t* src, int64_t region, int pos,
                              int kind, int lane, NewToken* nt = nullptr, const uint64_t* src_ll = nullptr,
                              uint32_t flag = 0, unsigned* sync_err = nullptr) {
  float x0, x1;
  if (COH) {
    uint32_t d0, d1;
    poll_pair<HD>(src_ll, lane, flag, sync_err, kv.err_word, d0, d1);
    x0 = bf16_to_f32((uint16_t)d0);
    x1 = (HD == 128) ? bf16_to_f32((uint16_t)d1) : 0.f;
  } else {
    x0 = bf16_to_f32(src[lane]);
    x1 = (HD == 128) ? bf16_to_f32(src[lane + 64]) : 0.f;
  }
  // FWHT, stages h = 1 .. 32 across lanes, then h = 64 inside the lane
#pragma unroll
  for (int h = 1; h < 64 && h < HD; h <<= 1) {
    const float p0 = lane_xor(x0, h, lane);
    x0 = (lane & h) ? (p0 - x0) : (x0 + p0);
    if (HD == 128) {
      const float p1 = lane_xor(x1, h, lane);
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
  const int64_t slot = region + pos;
  if (kind == 0) {
    // key slot: dword d = jj*(HD/32) + kb holds channels 32kb + 8jj + e
    uint32_t word = 0;
    const int d = lane;
    const int jj = d / (HD / 32), kb = d % (HD / 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 32 * kb + 8 * jj + e;
      const int v0 = __shfl(u0, c & 63, 64);
      const int v1 = __shfl(u1, c & 63, 64);
      word |= (uint32_t)((c < 64) ? v0 : v1) << (4 * nibble_slot(e));
    }
    if (d < HD / 8) reinterpret_cast<uint32_t*>(kv.k_codes + (size_t)slot * (HD / 2))[d] = word;
    if (lane == 0) kv.k_scales[slot] = s16;
    if (nt) {
      if (d < HD / 8) nt->kw[d] = word;
      if (lane == 0) nt->ks = s16;
    }
  } else {
    // value block: token w of the block sits in slot group jj, slot e
    const int w = pos % kVBlock;
    const int jj = (w % 16) / 4;
    const int e = (w % 4) + (w >= 16 ? 4 : 0);
    const int sh = 4 * nibble_slot(e);
    uint32_t* blk = kv.v_codes + (size_t)(region / kVBlock + pos / kVBlock) * 4 * HD;
#pragma unroll
    for (int q = 0; q < HD / 64; ++q) {
      const int c = lane + 64 * q;
      uint32_t* dw = blk + jj * HD + (c % 16) * (HD / 16) + c / 16;
      atomicAnd(dw, ~(0xFu << sh));
      atomicOr(dw, (uint32_t)(q ? u1 : u0) << sh);
      if (nt) nt->v[c] = (uint8_t)(q ? u1 : u0);
    }
    if (lane == 0) kv.v_scales[slot] = s16;
    if (nt && lane == 0) nt->vs = s16;
  }
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------

constexpr float kTwo24 = 16777216.0f;
__device__ __forceinline__ bool slot16(int e) { return (e & 2) != 0; }

// value of lane (l & ~15) | ((l + 8) & 15): the other half of a 16-lane row
__device__ __forceinline__ float dpp_row_ror8(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
}

template <int HD>
struct BlockRegs {
  uint32_t kw[2][HD / 32];  // key codes, 2 tiles of 16 tokens
  uint32_t vw[HD / 16];     // value codes, one dword per 16-channel block
  u32x2_t ks[2], vs[2];     // 4 fp16 scales per tile
};

template <int HD>
__device__ __forceinline__ void load_keys(BlockRegs<HD>& b, const uint8_t* kbase, const uint16_t* ksc,
                                          int blk, int c, int jj) {
  const int t0 = blk * kVBlock;
#pragma unroll
  for (int tile = 0; tile < 2; ++tile) {
    const uint8_t* kp = kbase + (size_t)(t0 + 16 * tile + c) * (HD / 2) + jj * (HD / 8);
    if (HD == 128) {
      const u32x4_t v = load16(kp);
      b.kw[tile][0] = v.x;
      b.kw[tile][1] = v.y;
      b.kw[tile][2] = v.z;
      b.kw[tile][3] = v.w;
    } else {
      const u32x2_t v = *reinterpret_cast<const u32x2_t*>(kp);
      b.kw[tile][0] = v.x;
      b.kw[tile][1] = v.y;
    }
    b.ks[tile] = *reinterpret_cast<const u32x2_t*>(ksc + t0 + 16 * tile + 4 * jj);
  }
}

template <int HD>
__device__ __forceinline__ void load_values(BlockRegs<HD>& b, const uint32_t* vbase, const uint16_t* vsc,
                                            int blk, int c, int jj) {
  constexpr int CB = HD / 16;
  const int t0 = blk * kVBlock;
#pragma unroll
  for (int tile = 0; tile < 2; ++tile)
    b.vs[tile] = *reinterpret_cast<const u32x2_t*>(vsc + t0 + 16 * tile + 4 * jj);
  const uint32_t* vp = vbase + (size_t)blk * 4 * HD + jj * HD + c * CB;
#pragma unroll
  for (int q = 0; q < CB / 4; ++q) {
    const u32x4_t v = load16(vp + 4 * q);
    b.vw[4 * q + 0] = v.x;
    b.vw[4 * q + 1] = v.y;
    b.vw[4 * q + 2] = v.z;
    b.vw[4 * q + 3] = v.w;
  }
}

template <int HD>
__device__ __forceinline__ void load_block(BlockRegs<HD>& b, const uint8_t* kbase, const uint32_t* vbase,
                                           const uint16_t* ksc, const uint16_t* vsc, int blk, int c,
                                           int jj) {
  load_keys<HD>(b, kbase, ksc, blk, c, jj);
  load_values<HD>(b, vbase, vsc, blk, c, jj);
}

// Put token w (0..31) of a block, read before that token was appended, into
// the block's registers from the append's LDS copy: the key words sit in
// the 16-lane row c == w % 16 of tile w / 16; the value nibble and both
// scales in the lanes of quarter jj == (w % 16) / 4.
template <int HD>
__device__ __forceinline__ void patch_new_token(BlockRegs<HD>& b, const NewToken& nt, int w, int c, int jj) {
  constexpr int KB = HD / 32, CB = HD / 16;
  const int tile = w / 16, tc = w % 16;
  if (c == tc) {
    uint32_t kw[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) kw[kb] = nt.kw[jj * KB + kb];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) b.kw[t][kb] = (t == tile) ? kw[kb] : b.kw[t][kb];
  }
  if (jj == tc / 4) {
    const int i = tc % 4;
    const int sh = 4 * nibble_slot(i + 4 * tile);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      b.vw[cb] = (b.vw[cb] & ~(0xFu << sh)) | ((uint32_t)nt.v[16 * cb + c] << sh);
    const uint32_t hs = 16u * (i & 1);
    const uint32_t keep = ~(0xFFFFu << hs);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (t == tile && q == (i >> 1)) {
          b.ks[t][q] = (b.ks[t][q] & keep) | ((uint32_t)nt.ks << hs);
          b.vs[t][q] = (b.vs[t][q] & keep) | ((uint32_t)nt.vs << hs);
        }
  }
}

__device__ __forceinline__ float f16_half(const u32x2_t& w, int i) {
  const uint32_t word = w[i >> 1];
  return f16_bits_to_f32((uint16_t)((i & 1) ? (word >> 16) : (word & 0xffffu)));
}

// inverse rotation of one head held by a wave (channels lane, lane + 64), / HD
template <int HD>
__device__ __forceinline__ void inverse_rotate(float& o0, float& o1, int lane) {
#pragma unroll
  for (int h = 1; h < 64 && h < HD; h <<= 1) {
    const float p0 = lane_xor(o0, h, lane);
    o0 = (lane & h) ? (p0 - o0) : (o0 + p0);
    if (HD == 128) {
      const float p1 = lane_xor(o1, h, lane);
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
}

// normalise, undo the rotation and store one head (one wave)
template <int HD, bool COH = false>
__device__ __forceinline__ void finish_head(const AttnArgs& a, size_t head_row, float lsum, float o0,
                                            float o1, int lane) {
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  o0 *= inv;
  o1 *= inv;
  inverse_rotate<HD>(o0, o1, lane);
  const size_t base = head_row * HD;
  if (a.attn_f32) {
    a.attn_f32[base + lane] = o0;
    if (HD == 128) a.attn_f32[base + lane + 64] = o1;
  }
  if (COH) {
    st_coh(&a.attn_bf16[base + lane], f32_to_bf16(o0));
    if (HD == 128) st_coh(&a.attn_bf16[base + lane + 64], f32_to_bf16(o1));
  } else {
    a.attn_bf16[base + lane] = f32_to_bf16(o0);
    if (HD == 128) a.attn_bf16[base + lane + 64] = f32_to_bf16(o1);
  }
}

// FWHT of one head (fp32, unnormalised) by one wave: channels lane and
// lane + 64 in registers, stages h = 1 .. 32 across lanes, h = 64 in-lane.
template <int HD>
__device__ __forceinline__ void fwht_wave(float& x0, float& x1, int lane) {
#pragma unroll
  for (int h = 1; h < 64 && h < HD; h <<= 1) {
    const float p0 = lane_xor(x0, h, lane);
    x0 = (lane & h) ? (p0 - x0) : (x0 + p0);
    if (HD == 128) {
      const float p1 = lane_xor(x1, h, lane);
      x1 = (lane & h) ? (p1 - x1) : (x1 + p1);
    }
  }
  if (HD == 128) {
    const float s0 = x0 + x1, s1 = x0 - x1;
    x0 = s0;
    x1 = s1;
  }
}

// One (row m, kv head j, split s) unit by one workgroup of NWA waves taking
// interleaved 32-token blocks of the split.  `wait_input` runs after the
// first cache loads are issued and before the query is read.  LDS: wm, wl
// [NWA][8], wo [NWA][8][HD], then the query operand (attn_lds_floats).
// COH: the query and the new key/value come from other workgroups of the
// same launch as flagged words (polled loads); the partials are exchanged
// with agent-coherent stores and loads.
// Row metadata of a unit read ahead of time (the one-launch step reads it
// at its start, so that the read is not on the attention critical path).
struct RowMeta {
  int64_t base, cap;
  int L;
};

// LDS of attn_body in floats: wm, wl [NWA][8], wo [NWA][8][HD], the query
// operand halves [2][8][HD] fp16 and their sums [8][2], the appended token
template <int HD, int NWA>
__host__ __device__ constexpr int attn_lds_floats() {
  return 2 * NWA * 8 + NWA * 8 * HD + 8 * HD + 16 + (int)(sizeof(NewToken) + 3) / 4;
}

template <int HD, int NWA, bool COH, typename Wait>
__device__ __forceinline__ void attn_body(const AttnArgs& a, const int m, const int j, const int s, float* lds,
                                          Wait&& wait_input, const RowMeta* meta = nullptr) {
  constexpr int KB = HD / 32;  // 32-channel MFMA steps for q.k
  constexpr int CB = HD / 16;  // 16-channel output blocks
  constexpr int GMAX = 8;
  float (*wm)[GMAX] = reinterpret_cast<float (*)[GMAX]>(lds);
  float (*wl)[GMAX] = reinterpret_cast<float (*)[GMAX]>(lds + NWA * GMAX);
  float (*wo)[GMAX][HD] = reinterpret_cast<float (*)[GMAX][HD]>(lds + 2 * NWA * GMAX);
  // the rotated queries as the fp16 operand of q.k: high and low halves
  // [GMAX][HD] each, and per (head, half) 8 * the sum of the values the
  // half represents
  uint16_t (*qh)[HD] = reinterpret_cast<uint16_t (*)[HD]>(lds + 2 * NWA * GMAX + NWA * GMAX * HD);
  uint16_t (*ql)[HD] = qh + GMAX;
  float (*cqs)[2] = reinterpret_cast<float (*)[2]>(ql + GMAX);
  NewToken* nt = reinterpret_cast<NewToken*>(cqs + GMAX);

  const KvArgs& kv = a.kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, jj = lane >> 4;
  const int S = a.S, G = a.G;

  const int64_t base = meta ? meta->base : kv.row_base[m];
  const int64_t cap = meta ? meta->cap : kv.row_base[m + 1] - base;
  // the splits partition [0, S bps) blocks (sized for the longest row): a
  // shorter row leaves its last splits empty
  const int bps = a.bps;
  int L = meta ? meta->L : a.ctx_len[m];
  const bool len_ok = L >= 1 && L <= cap && L <= S * bps * kVBlock;
  if (!len_ok) {
    if (tid == 0 && kv.err_word) atomicOr(kv.err_word, I4D_DEVERR_CTX_LEN);
    L = (int)max((int64_t)0, min((int64_t)max(L, 1), min(cap, (int64_t)S * bps * kVBlock)));
  }
  const int nblk = (L + kVBlock - 1) / kVBlock;
  const int b0 = s * bps;
  const int b1 = min(nblk, b0 + bps);
  const int64_t region = base * kv.n_kv + (int64_t)j * cap;
  const uint8_t* kbase = kv.k_codes + (size_t)region * (HD / 2);
  const uint16_t* ksc = kv.k_scales + region;
  const uint16_t* vsc = kv.v_scales + region;
  const uint32_t* vbase = kv.v_codes + (size_t)(region / kVBlock) * 4 * HD;
  // every load of the kernel is issued unconditionally (a wave without work
  // reads a valid block it then ignores), so the compiler can wait on exact
  // load counts instead of draining all loads at control-flow joins
  const int last_valid = max(b1, 1) - 1;  // block 0 exists: capacity >= 32

  // In a decode step the split holding position L-1 first appends the new
  // key/value there.  Cache reads do not depend on the query, so every wave
  // starts loading its first block now; the block being appended to is
  // read before the append and the new token put into its registers after.
  const int last_blk = (L - 1) / kVBlock;
  const bool appending = a.k_new && len_ok && last_blk >= b0 && last_blk < b1;
  // Stand-alone: two blocks per wave in flight (its first two, then two
  // ahead of the one being consumed).  In the one-launch step a split has
  // about one block per wave: one in flight.
  constexpr bool TWO = !COH;
  int blk = b0 + wave;
  BlockRegs<HD> cur, nxt;
  load_block<HD>(cur, kbase, vbase, ksc, vsc, min(blk, last_valid), c, jj);
  if (TWO) load_block<HD>(nxt, kbase, vbase, ksc, vsc, min(blk + NWA, last_valid), c, jj);
  // the query and the new key/value may come from other workgroups of the
  // same launch: wait for them only now
  wait_input();

  // The score scale enters q.k in two parts: qs in [1, 2) with the query
  // and the power of two unq = score_scale / qs after the product.
  int sk = 0;
  const float qs = 2.0f * frexpf(a.score_scale, &sk);
  const float unq = ldexpf(1.0f, sk - 1);
  // rotate the G query heads of this kv head (one wave per head) and store
  // them as the partner operand of q.k: channel ch as w = q * qs (and 1/16
  // at ch % 8 in {2,3,6,7}, the slots paired with a high nibble) split into
  // the fp16 high part fp16(w) and the low part fp16(w - high); per half
  // the sum of 8 (128 at the 1/16 slots) times its values (the code offset
  // term)
  for (int g = wave; g < G; g += NWA) {
    float x0, x1;
    if (COH) {
      uint32_t d0, d1;
      poll_pair<HD>(a.q_ll + ((size_t)j * G + g) * HD, lane, a.flag, a.sync_err, kv.err_word, d0, d1);
      x0 = __uint_as_float(d0);
      x1 = (HD == 128) ? __uint_as_float(d1) : 0.f;
    } else {
      const float* src = a.q + ((size_t)m * a.n_q + (size_t)j * G + g) * HD;
      x0 = src[lane];
      x1 = (HD == 128) ? src[lane + 64] : 0.f;
    }
    fwht_wave<HD>(x0, x1, lane);
    float sh = 0.f, sl = 0.f;
    auto put = [&](const float x, const int ch) {
      const bool s16 = slot16(ch & 7);
      const float w = x * (s16 ? qs * 0.0625f : qs);
      const _Float16 hi = (_Float16)w;
      const _Float16 lo = (_Float16)(w - (float)hi);
      qh[g][ch] = bitcast<uint16_t>(hi);
      ql[g][ch] = bitcast<uint16_t>(lo);
      sh = fmaf((float)hi, s16 ? 128.f : 8.f, sh);
      sl = fmaf((float)lo, s16 ? 128.f : 8.f, sl);
    };
    put(x0, lane);
    if (HD == 128) put(x1, lane + 64);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      sh += lane_xor(sh, off, lane);
      sl += lane_xor(sl, off, lane);
    }
    if (lane == 0) {
      cqs[g][0] = sh;
      cqs[g][1] = sl;
    }
  }
  // the append by two waves that rotate no query head, where there are two
  const int aw = (G + 2 <= NWA) ? G : 0;
  if (appending && wave >= aw && wave < aw + 2) {
    const uint16_t* src = (wave - aw ? a.v_new : a.k_new) + ((size_t)m * kv.n_kv + j) * HD;
    append_vector<HD, COH>(kv, src, region, L - 1, wave - aw, lane, nt,
                           COH ? (wave - aw ? a.v_ll : a.k_ll) + (size_t)j * HD : nullptr, a.flag, a.sync_err);
    // the new codes are in memory before a block read of this workgroup
    // after the first (two) per wave, if one of those is the block appended to
    if (last_blk >= b0 + (TWO ? 2 : 1) * NWA) wait_vmem();
  }
  lds_barrier();

  // Rotated query as the partner operand of q.k: columns c < 8 hold the
  // high fp16 part of query head j*G + c (c < G), columns 8 + c the low part
  // (the residual).  cq: the code offset term of column c, times unq.
  f16x8_t qop[KB];
  float cq;
  {
    const int head = c & 7;
    const bool active = head < G;
    const uint16_t* qsrc = (c >= 8 ? ql : qh)[head];
    const f16x8_t zero = {};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const f16x8_t v = *reinterpret_cast<const f16x8_t*>(&qsrc[32 * kb + 8 * jj]);
      qop[kb] = active ? v : zero;
    }
    const float t = cqs[head][c >= 8 ? 1 : 0];
    cq = active ? t * unq : 0.f;
  }
  if (appending) {
    const int w = (L - 1) % kVBlock;
    if (blk == last_blk) patch_new_token<HD>(cur, *nt, w, c, jj);
    if (TWO && blk + NWA == last_blk) patch_new_token<HD>(nxt, *nt, w, c, jj);
  }

  float m_run = -INFINITY, l_run = 0.f;
  // per column c, the sum of the fp16 p' values (times 16 at the slots
  // paired with a high nibble) over the tokens so far: one MFMA per block
  // with a constant partner operand, so every row holds the column total
  f32x4_t psv = {0.f, 0.f, 0.f, 0.f};
  const float accf = kTwo24 * unq;  // undo the 2^-24 of the code operand and qs
  const _Float16 h1 = (_Float16)1.0f, h16 = (_Float16)16.0f;
  const f16x8_t pones = {h1, h1, h16, h16, h1, h1, h16, h16};
  f32x4_t o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Blocks in registers (cur, and nxt when two are in flight): once a
  // block's keys are consumed, the keys of the wave's block one (two) ahead
  // are requested into them, its values likewise once the values are.  The
  // wave's last block(s) run the same body without those requests and with
  // the token mask (only the row's last block can be partial, and it is the
  // last block of its wave; its slots past L may hold anything).
  // Columns c >= G carry finite values that no output uses.
  auto body = [&](BlockRegs<HD>& cur, const int bcur, const int nb, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    const int t0 = bcur * kVBlock;
    float sc[8];
    float mx = -INFINITY;
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dword_to_f16x8_sub(cur.kw[tile][kb]), qop[kb], acc,
                                                     0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // high part (column c) + low part (column c + 8, rotated in by DPP)
        const float part = fmaf(acc[i], accf, -cq);
        const float full = part + dpp_row_ror8(part);
        // scale products as FMAs with the fp16 scale as a mixed-precision
        // operand (one v_fma_mix instead of a conversion and a multiply)
        float v = fmaf(full, f16_half(cur.ks[tile], i), 0.0f);
        if (LAST) v = (t0 + 16 * tile + 4 * jj + i < L) ? v : -INFINITY;
        sc[tile * 4 + i] = v;
      }
    }
    if (!LAST) load_keys<HD>(cur, kbase, ksc, nb, c, jj);
    mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mx = fmaxf(mx, lane_xor(mx, 16, lane));
    mx = fmaxf(mx, lane_xor(mx, 32, lane));
    const float m_new = fmaxf(m_run, mx);  // finite: the block holds a valid token
    // rescale only when some column's running maximum moved (alpha = 1
    // exactly elsewhere)
    if (__any(m_new > m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      psv *= alpha;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) o[cb] *= alpha;
    }
    // P operand: element e is token 4jj+e (e < 4) or 16+4jj+e-4 (e >= 4),
    // i.e. score register e; value scale folded in, 1/16 at e in {2,3,6,7}
    f16x8_t pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tile = e >> 2, i = e & 3;
      const float p = __builtin_amdgcn_exp2f(sc[e] - m_new);  // 0 for masked tokens
      l_run += p;
      float pv = fmaf(p, f16_half(cur.vs[tile], i), 0.0f);
      if (slot16(e)) pv *= 0.0625f;
      if (LAST) pv = (p > 0.f) ? pv : 0.f;
      const _Float16 ph = (_Float16)pv;
      pb[e] = ph;
    }
    psv = __builtin_amdgcn_mfma_f32_16x16x32_f16(pones, pb, psv, 0, 0, 0);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dword_to_f16x8_sub(cur.vw[cb]), pb, o[cb], 0, 0, 0);
    if (!LAST) load_values<HD>(cur, vbase, vsc, nb, c, jj);
    m_run = m_new;
  };
  if (blk < b1) {
    if constexpr (TWO) {
      const int nbw = (b1 - 1 - blk) / NWA + 1;  // blocks of this wave
      int i = 0;
      for (; i + 2 < nbw; i += 2) {
        body(cur, blk, min(blk + 2 * NWA, last_valid), std::false_type());
        body(nxt, blk + NWA, min(blk + 3 * NWA, last_valid), std::false_type());
        blk += 2 * NWA;
      }
      body(cur, blk, 0, std::true_type());
      if (i + 2 == nbw) body(nxt, blk + NWA, 0, std::true_type());
    } else {
      for (; blk + NWA < b1; blk += NWA) body(cur, blk, blk + NWA, std::false_type());
      body(cur, blk, 0, std::true_type());
    }
  }

  // per-column totals over the 4 lane quarters; undo the 2^-24 operand
  // scale and remove the code offset: o = 2^24 acc - 8 * sum p'
  l_run += lane_xor(l_run, 16, lane);
  l_run += lane_xor(l_run, 32, lane);
  const float vbias = 8.f * psv[0];
  if (c < G) {
    if (jj == 0) {
      wm[wave][c] = m_run;
      wl[wave][c] = l_run;
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) wo[wave][c][16 * cb + 4 * jj + i] = fmaf(o[cb][i], kTwo24, -vbias);
  }
  __syncthreads();

  // wave w merges heads w, w + NWA, ... over the waves (every LDS read of
  // the merge issued at once; a wave without tokens has sum 0)
  for (int g = wave; g < G; g += NWA) {
    float mw[NWA], lw[NWA], p0[NWA], p1[NWA];
#pragma unroll
    for (int w = 0; w < NWA; ++w) {
      mw[w] = wm[w][g];
      lw[w] = wl[w][g];
      p0[w] = wo[w][g][lane];
      p1[w] = (HD == 128) ? wo[w][g][lane + 64] : 0.f;
    }
    float M_ = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWA; ++w) M_ = lw[w] > 0.f ? fmaxf(M_, mw[w]) : M_;
    float lsum = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int w = 0; w < NWA; ++w) {
      if (lw[w] > 0.f) {
        const float f = exp2f(mw[w] - M_);
        lsum += f * lw[w];
        o0 += f * p0[w];
        o1 += f * p1[w];
      }
    }
    const size_t head_row = (size_t)m * a.n_q + (size_t)j * G + g;
    if (S == 1) {
      finish_head<HD, COH>(a, head_row, lsum, o0, o1, lane);
    } else {
      const size_t ph = head_row * S + s;
      if (COH) {
        st_coh(&a.part_o[ph * HD + lane], o0);
        if (HD == 128) st_coh(&a.part_o[ph * HD + lane + 64], o1);
        if (lane == 0) {
          st_coh(&a.part_ml[ph * 2], M_);
          st_coh(&a.part_ml[ph * 2 + 1], lsum);
        }
      } else {
        a.part_o[ph * HD + lane] = o0;
        if (HD == 128) a.part_o[ph * HD + lane + 64] = o1;
        if (lane == 0) {
          a.part_ml[ph * 2] = M_;
          a.part_ml[ph * 2 + 1] = lsum;
        }
      }
    }
  }
}

// Merge the splits of one (row, q head) and undo the rotation:
// o = H o~ / hd with o~ = sum_s e^(m_s - m) o~_s / sum_s e^(m_s - m) l_s.
// One wave per (row, head); lane t holds split t (t + 64, ...) for the
// weights, the partial outputs are read with independent loads.
template <int HD, bool COH = false>
__device__ __forceinline__ void combine_head(const AttnArgs& a, size_t head_row, int lane, float& lsum_out,
                                             float& o0_out, float& o1_out) {
  auto ld = [](const float* p) { return COH ? ld_coh(p) : *p; };
  constexpr int CH = 32;  // splits whose partial outputs are in flight at once
  const int S = a.S;
  const float* ml = a.part_ml + head_row * S * 2;
  const float* po = a.part_o + head_row * S * HD;
  // one round trip per 32 splits: the chunk's (max, sum) pairs (lane u < CH
  // holds split t0 + u) and its partial outputs are requested together;
  // the running maximum is rescaled per chunk
  float M_ = -INFINITY, lsum = 0.f, o0 = 0.f, o1 = 0.f;
  const int nch = (S + CH - 1) / CH;
  for (int c = 0; c < nch; ++c) {
    const int t0 = c * CH;
    const int tl = min(t0 + (lane & (CH - 1)), S - 1);
    const float mt = ld(&ml[2 * tl]);
    const float lt = ld(&ml[2 * tl + 1]);
    float x0[CH], x1[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int t = min(t0 + u, S - 1);
      x0[u] = ld(&po[(size_t)t * HD + lane]);
      x1[u] = (HD == 128) ? ld(&po[(size_t)t * HD + lane + 64]) : 0.f;
    }
    // an empty split has sum 0 and contributes nothing
    const bool valid = (lane < CH) && (t0 + lane < S) && lt > 0.f;
    const float mc = wave_max(valid ? mt : -INFINITY);
    const float M_new = fmaxf(M_, mc);
    if (M_new > -INFINITY) {
      const float alpha = exp2f(M_ - M_new);  // 0 while M_ is -inf
      lsum *= alpha;
      o0 *= alpha;
      o1 *= alpha;
      const float f = valid ? exp2f(mt - M_new) : 0.f;
      lsum = fmaf(f, valid ? lt : 0.f, lsum);
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const float fu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), u));
        o0 = fmaf(fu, x0[u], o0);
        o1 = fmaf(fu, x1[u], o1);
      }
      M_ = M_new;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lsum += lane_xor(lsum, off, lane);
  lsum_out = lsum;
  o0_out = o0;
  o1_out = o1;
}

}  // namespace i4d
