// api_host.cpp - host-only part of the C ABI: errors, sizes, weight packing,
// cache decoding for tests, workspace layouts.  No GPU calls here.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <string>
#include <thread>
#include <vector>

#include "i4d_internal.h"

namespace i4d {

static thread_local std::string g_err;

i4d_status fail(i4d_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

i4d_status ok() { return I4D_OK; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

i4d_status check_shape(const i4d_layer_shape* s) {
  if (!s) return fail(I4D_ERR_NULL, "layer shape is NULL");
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(I4D_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", s->head_dim);
  if (s->hadamard_block != s->head_dim)
    return fail(I4D_ERR_UNSUPPORTED, "hadamard_block %d must equal head_dim %d", s->hadamard_block,
                s->head_dim);
  if (s->group != kGroup) return fail(I4D_ERR_UNSUPPORTED, "group %d must be 128", s->group);
  if (s->n_q_heads <= 0 || s->n_kv_heads <= 0 || s->n_q_heads % s->n_kv_heads)
    return fail(I4D_ERR_SHAPE, "n_q_heads %d must be a positive multiple of n_kv_heads %d",
                s->n_q_heads, s->n_kv_heads);
  int G = s->n_q_heads / s->n_kv_heads;
  if (G > 8 || (G & (G - 1)))
    return fail(I4D_ERR_UNSUPPORTED, "GQA group %d must be a power of two <= 8", G);
  int dims[3] = {s->d_model, s->n_q_heads * s->head_dim, s->d_ffn};
  for (int d : dims)
    if (d <= 0 || d % kGroup)
      return fail(I4D_ERR_SHAPE, "dimension %d must be a positive multiple of 128", d);
  if (!(s->rms_eps > 0.f) || !(s->rope_theta > 1.f))
    return fail(I4D_ERR_RANGE, "rms_eps must be > 0 and rope_theta > 1");
  return ok();
}

AttnPlan attn_plan(const i4d_layer_shape* s, int M, int max_ctx_len, int num_splits) {
  // One workgroup per (row, kv head, split); every split spans the same
  // number of blocks (sized by max_ctx_len), so a short row leaves splits
  // empty.  Automatic split count: about one workgroup per CU (256) over
  // all (row, kv head) pairs, at least 4 blocks of 32 tokens per split
  // (more, shorter splits measured slower: per-split setup, the merge and
  // the combine launch outweigh the better balance of ragged rows).  Then
  // 4 or 8 waves per workgroup (8 while every wave keeps two blocks or more
  // and the launch has fewer than 4096 waves; each wave holds two blocks in
  // registers, which 16 waves would not fit).
  const long nblk = (max_ctx_len + kVBlock - 1) / kVBlock;
  const long units = (long)M * s->n_kv_heads;
  long S;
  if (num_splits > 0) {
    S = std::min(num_splits, I4D_MAX_SPLITS);
  } else {
    S = (256 + units - 1) / units;
    S = std::min<long>(S, std::max<long>(1, nblk / 4));
    S = std::max<long>(std::min<long>(S, I4D_MAX_SPLITS), 1);
  }
  const long bps = (nblk + S - 1) / S;
  int nwa = 4;
  if (units * S * 8 < 4096 && bps >= 16) nwa = 8;
  AttnPlan p;
  p.S = (int)S;
  p.nwa = nwa;
  return p;
}

int step_m1_splits(const i4d_layer_shape* s, int max_ctx_len, int num_splits) {
  if (num_splits > 0) return std::min(num_splits, I4D_MAX_SPLITS);
  const int nblk = (max_ctx_len + kVBlock - 1) / kVBlock;
  return std::max(1, std::min(256 / s->n_kv_heads, nblk));
}

AttnWs attn_ws_layout(const i4d_layer_shape* s, int M, int S) {
  AttnWs w;
  size_t n = (size_t)M * s->n_q_heads * S;
  w.ml = 0;
  w.o = align256(n * 2 * sizeof(float));
  w.total = w.o + align256(n * s->head_dim * sizeof(float));
  return w;
}

StepLl step_ll_layout(const i4d_layer_shape* s) {
  StepLl w;
  const size_t nq = (size_t)s->n_q_heads * s->head_dim, nk = (size_t)s->n_kv_heads * s->head_dim;
  size_t off = 0;
  w.q = off;    off += align256(nq * 8);
  w.k = off;    off += align256(nk * 8);
  w.v = off;    off += align256(nk * 8);
  w.total = off;
  return w;
}

LmWs lm_ws_layout(int V, int M) {
  LmWs w;
  int strips = V / kStrip;
  w.nwaves = (strips + kLmStripsPerWave - 1) / kLmStripsPerWave;
  w.val = 0;
  w.idx = align256((size_t)w.nwaves * M * sizeof(float));
  w.total = w.idx + align256((size_t)w.nwaves * M * sizeof(int32_t));
  return w;
}

// ---------------------------------------------------------------------------
// fp16 / bf16 conversions (host)
// ---------------------------------------------------------------------------

static inline uint16_t f32_to_f16_sat(float f) {
  _Float16 h = (_Float16)f;  // IEEE round-to-nearest-even
  uint16_t b;
  memcpy(&b, &h, 2);
  if ((b & 0x7fffu) == 0x7c00u && isfinite(f)) b = (uint16_t)((b & 0x8000u) | 0x7bffu);
  return b;
}

static inline float f16_to_f32(uint16_t b) {
  _Float16 h;
  memcpy(&h, &b, 2);
  return (float)h;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// symmetric INT4 RTN of one 128-wide group: scale fp16(absmax/7), codes in [-8, 7]
static inline uint16_t quantize_group(const float* w, int8_t* q) {
  float a = 0.f;
  for (int k = 0; k < kGroup; ++k) a = std::max(a, fabsf(w[k]));
  uint16_t s16 = f32_to_f16_sat(a / 7.0f);
  float sf = f16_to_f32(s16);
  for (int k = 0; k < kGroup; ++k) {
    if (sf == 0.f) {
      q[k] = 0;
    } else {
      float r = rintf(w[k] / sf);
      r = std::min(7.f, std::max(-8.f, r));
      q[k] = (int8_t)r;
    }
  }
  return s16;
}

// E4M3 (OCP FP8: 4 exponent bits, bias 7, 3 mantissa bits, largest finite
// 448) of a finite fp32 value: nearest, ties to the even mantissa, 448 and
// above saturating to 448; the sign is kept (also on zero)
static inline uint8_t e4m3_of(float x) {
  const uint8_t sign = std::signbit(x) ? 0x80 : 0x00;
  const double a = fabs((double)x);
  if (!(a < 448.0)) return sign | 0x7E;
  if (a < 0.015625) return sign | (uint8_t)nearbyint(a * 512.0);  // 2^-9 steps; 8 -> 2^-6 = 0x08
  int e;
  frexp(a, &e);                          // a in [2^(e-1), 2^e)
  double q = nearbyint(ldexp(a, 4 - e));  // mantissa steps of 2^(e-4): 8..16
  int E = e - 1;
  if (q >= 16.0) {
    q = 8.0;
    ++E;
  }
  const int code = ((E + 7) << 3) | ((int)q - 8);
  return sign | (uint8_t)std::min(code, 0x7E);
}

// E4M3 codes of one 128-wide group: scale fp16(absmax / 448)
static inline uint16_t quantize_group_e4m3(const float* w, uint8_t* q) {
  float a = 0.f;
  for (int k = 0; k < kGroup; ++k) a = std::max(a, fabsf(w[k]));
  const uint16_t s16 = f32_to_f16_sat(a / 448.0f);
  const float sf = f16_to_f32(s16);
  for (int k = 0; k < kGroup; ++k) q[k] = sf == 0.f ? 0 : e4m3_of(w[k] / sf);
  return s16;
}

// the smallest e with absmax <= 448 * 2^e: with absmax = m 2^x (0.5 <= m < 1)
// and 448 = 0.875 2^9 that is x - 9 when m <= 0.875, else x - 8; clamped to
// the E8M0 range [-127, 127]; an all-zero group takes -127
static inline int mx_exponent_of(float a) {
  if (a == 0.f) return -127;
  int x;
  const double m = frexp((double)a, &x);
  const int e = (m <= 0.875) ? x - 9 : x - 8;
  return std::min(127, std::max(-127, e));
}

// E4M3 codes of one 128-wide group with a power-of-two scale 2^e: codes of
// w * 2^-e (exact scaling, no saturation); returns the E8M0 byte e + 127
static inline uint8_t quantize_group_mx(const float* w, uint8_t* q) {
  float a = 0.f;
  for (int k = 0; k < kGroup; ++k) a = std::max(a, fabsf(w[k]));
  const int e = mx_exponent_of(a);
  for (int k = 0; k < kGroup; ++k) q[k] = e4m3_of((float)ldexp((double)w[k], -e));
  return (uint8_t)(e + 127);
}

template <typename F>
static void parallel_for(long n, int threads, F&& fn) {
  if (threads <= 0) threads = (int)std::max(1u, std::thread::hardware_concurrency());
  threads = (int)std::min<long>(threads, std::max<long>(1, n));
  if (threads == 1) {
    fn(0L, n);
    return;
  }
  std::vector<std::thread> pool;
  long chunk = (n + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    long lo = t * chunk, hi = std::min(n, lo + chunk);
    if (lo >= hi) break;
    pool.emplace_back([&fn, lo, hi] { fn(lo, hi); });
  }
  for (auto& th : pool) th.join();
}

static i4d_status check_pack_args(i4d_proj_kind kind, int N, int K, int head_dim) {
  if (N <= 0 || K <= 0 || K % kGroup)
    return fail(I4D_ERR_SHAPE, "K=%d must be a positive multiple of 128 (N=%d)", K, N);
  if (N % kStrip) return fail(I4D_ERR_SHAPE, "N=%d must be a multiple of 16", N);
  if (kind == I4D_PROJ_QKV) {
    if (head_dim != 64 && head_dim != 128)
      return fail(I4D_ERR_UNSUPPORTED, "QKV head_dim %d must be 64 or 128", head_dim);
    if (N % head_dim) return fail(I4D_ERR_SHAPE, "QKV N=%d not a multiple of head_dim", N);
  } else if (kind == I4D_PROJ_GATE_UP) {
    if (N % 8) return fail(I4D_ERR_SHAPE, "gate/up N=%d must be a multiple of 8", N);
  } else if (kind != I4D_PROJ_PLAIN) {
    return fail(I4D_ERR_RANGE, "unknown projection kind %d", (int)kind);
  }
  return ok();
}

static inline int packed_rows(i4d_proj_kind kind, int N) {
  return kind == I4D_PROJ_GATE_UP ? 2 * N : N;
}

// packed row p -> (matrix 0/1, logical row)
static inline void source_row(i4d_proj_kind kind, int p, int head_dim, int* mat, int* row) {
  if (kind == I4D_PROJ_QKV) {
    *mat = 0;
    *row = qkv_logical_row(p, head_dim);
  } else if (kind == I4D_PROJ_GATE_UP) {
    int t = p / kStrip, i = p % kStrip;
    *mat = i < 8 ? 0 : 1;
    *row = 8 * t + (i & 7);
  } else {
    *mat = 0;
    *row = p;
  }
}

}  // namespace i4d

using namespace i4d;

// E4M3 atoms with one scale per (row, group) of type S from quantize_group
template <typename S, typename QG>
static i4d_status pack_e4m3_atoms(i4d_proj_kind kind, const float* W0, const float* W1, const float* gamma, int N,
                                  int K, int head_dim, void* codes_out, S* scales_out, int threads, QG quantize_group) {
  i4d_status st = check_pack_args(kind, N, K, head_dim);
  if (st) return st;
  if (!W0 || !codes_out || !scales_out) return fail(I4D_ERR_NULL, "W0/codes_out/scales_out NULL");
  if (kind == I4D_PROJ_GATE_UP && !W1) return fail(I4D_ERR_NULL, "gate/up needs W1 (up)");
  if (kind == I4D_PROJ_PLAIN && gamma)
    return fail(I4D_ERR_RANGE, "PLAIN projections take no gain (gamma must be NULL)");
  const int Np = packed_rows(kind, N);
  const int G = groups_of(K);
  uint8_t* codes = (uint8_t*)codes_out;
  parallel_for(Np / kStrip, threads, [&](long t0, long t1) {
    float w[kGroup];
    uint8_t q[kGroup];
    for (long t = t0; t < t1; ++t) {
      for (int r = 0; r < kStrip; ++r) {
        int p = (int)t * kStrip + r, mat, row;
        source_row(kind, p, head_dim, &mat, &row);
        const float* src = (mat ? W1 : W0) + (size_t)row * K;
        for (int g = 0; g < G; ++g) {
          for (int k = 0; k < kGroup; ++k) {
            const float v = src[g * kGroup + k];
            w[k] = gamma ? gamma[g * kGroup + k] * v : v;  // one fp32 product
          }
          scales_out[((size_t)t * G + g) * kStrip + r] = quantize_group(w, q);
          for (int k = 0; k < kGroup; ++k) codes[e4m3_code_offset(p, g * kGroup + k, K)] = q[k];
        }
      }
    }
  });
  return ok();
}

template <typename S>
static i4d_status unpack_e4m3_atoms(i4d_proj_kind kind, const void* codes, const S* scales, int N, int K,
                                    int head_dim, uint8_t* q_out, S* s_out) {
  i4d_status st = check_pack_args(kind, N, K, head_dim);
  if (st) return st;
  if (!codes || !scales || !q_out || !s_out) return fail(I4D_ERR_NULL, "NULL pointer");
  const int Np = packed_rows(kind, N);
  const int G = groups_of(K);
  const uint8_t* c = (const uint8_t*)codes;
  for (int p = 0; p < Np; ++p) {
    int mat, row;
    source_row(kind, p, head_dim, &mat, &row);
    const int out_row = mat * N + row;
    for (int k = 0; k < K; ++k) q_out[(size_t)out_row * K + k] = c[e4m3_code_offset(p, k, K)];
    for (int g = 0; g < G; ++g) s_out[(size_t)out_row * G + g] = scales[scale_index(p, g, K)];
  }
  return ok();
}

extern "C" {

const char* i4d_last_error(void) { return g_err.c_str(); }

const char* i4d_version(void) { return "i4d 0.1 (gfx950)"; }

i4d_status i4d_packed_sizes(i4d_proj_kind kind, int N, int K, int head_dim, size_t* code_bytes,
                            size_t* scale_bytes) {
  if (!code_bytes || !scale_bytes) return fail(I4D_ERR_NULL, "output pointer is NULL");
  i4d_status st = check_pack_args(kind, N, K, head_dim);
  if (st) return st;
  int Np = packed_rows(kind, N);
  *code_bytes = packed_code_bytes(Np, K);
  *scale_bytes = packed_scale_elems(Np, K) * sizeof(uint16_t);
  return ok();
}

// the 128 codes q (in [-8, 7]) of packed row r (0..15) into the group's
// atom: nibble u = q + 8 of channel kk at lane (16 j + r), dword kb, slot
// nibble_slot(e) for kk = 32 kb + 8 j + e
static inline void place_group(uint8_t* atom, int r, const int8_t* q) {
  for (int kk = 0; kk < kGroup; ++kk) {
    const int kb = kk / 32, j = (kk % 32) / 8, e = kk % 8;
    const int slot = nibble_slot(e);
    const uint8_t u = (uint8_t)(q[kk] + 8);
    uint8_t* byte = atom + (16 * j + r) * 16 + kb * 4 + slot / 2;
    *byte |= (slot & 1) ? (uint8_t)(u << 4) : u;
  }
}

i4d_status i4d_pack_weights(i4d_proj_kind kind, const float* W0, const float* W1,
                            const float* gamma, int N, int K, int head_dim, void* codes_out,
                            uint16_t* scales_out, int threads) {
  i4d_status st = check_pack_args(kind, N, K, head_dim);
  if (st) return st;
  if (!W0 || !codes_out || !scales_out) return fail(I4D_ERR_NULL, "W0/codes_out/scales_out NULL");
  if (kind == I4D_PROJ_GATE_UP && !W1) return fail(I4D_ERR_NULL, "gate/up needs W1 (up)");
  if (kind == I4D_PROJ_PLAIN && gamma)
    return fail(I4D_ERR_RANGE, "PLAIN projections take no gain (gamma must be NULL)");
  const int Np = packed_rows(kind, N);
  const int G = groups_of(K);
  uint8_t* codes = (uint8_t*)codes_out;
  memset(scales_out, 0, packed_scale_elems(Np, K) * sizeof(uint16_t));
  parallel_for(Np / kStrip, threads, [&](long t0, long t1) {
    std::vector<float> w(kGroup);
    int8_t q[kGroup];
    for (long t = t0; t < t1; ++t) {
      uint8_t* atom_base = codes + (size_t)t * G * kAtomBytes;
      memset(atom_base, 0, (size_t)G * kAtomBytes);
      for (int r = 0; r < kStrip; ++r) {
        int p = (int)t * kStrip + r, mat, row;
        source_row(kind, p, head_dim, &mat, &row);
        const float* src = (mat ? W1 : W0) + (size_t)row * K;
        for (int g = 0; g < G; ++g) {
          for (int k = 0; k < kGroup; ++k) {
            float v = src[g * kGroup + k];
            w[k] = gamma ? gamma[g * kGroup + k] * v : v;  // one fp32 product
          }
          uint16_t s16 = quantize_group(w.data(), q);
          scales_out[((size_t)t * G + g) * kStrip + r] = s16;
          place_group(atom_base + (size_t)g * kAtomBytes, r, q);
        }
      }
    }
  });
  return ok();
}

i4d_status i4d_pack_codes(i4d_proj_kind kind, const int8_t* q, const uint16_t* s, int N, int K,
                          int head_dim, void* codes_out, uint16_t* scales_out, int threads) {
  i4d_status st = check_pack_args(kind, N, K, head_dim);
  if (st) return st;
  if (!q || !s || !codes_out || !scales_out) return fail(I4D_ERR_NULL, "q/s/codes_out/scales_out NULL");
  const int Np = packed_rows(kind, N);
  const int G = groups_of(K);
  const size_t rows = (size_t)Np;  // N, or 2N for gate/up
  // everything is checked before anything is written
  for (size_t i = 0; i < rows * (size_t)K; ++i)
    if (q[i] < -8 || q[i] > 7)
      return fail(I4D_ERR_RANGE, "code %d at row %zu, column %zu is outside [-8, 7]", (int)q[i], i / K, i % K);
  for (size_t i = 0; i < rows * (size_t)G; ++i)
    if ((s[i] & 0x7c00u) == 0x7c00u)
      return fail(I4D_ERR_RANGE, "scale of row %zu, group %zu is not finite (0x%04x)", i / G, i % G, s[i]);
  uint8_t* codes = (uint8_t*)codes_out;
  parallel_for(Np / kStrip, threads, [&](long t0, long t1) {
    for (long t = t0; t < t1; ++t) {
      uint8_t* atom_base = codes + (size_t)t * G * kAtomBytes;
      memset(atom_base, 0, (size_t)G * kAtomBytes);
      for (int r = 0; r < kStrip; ++r) {
        int p = (int)t * kStrip + r, mat, row;
        source_row(kind, p, head_dim, &mat, &row);
        const size_t in_row = (size_t)mat * N + row;
        for (int g = 0; g < G; ++g) {
          scales_out[((size_t)t * G + g) * kStrip + r] = s[in_row * G + g];
          place_group(atom_base + (size_t)g * kAtomBytes, r, q + in_row * K + (size_t)g * kGroup);
        }
      }
    }
  });
  return ok();
}

i4d_status i4d_packed_sizes_e4m3(i4d_proj_kind kind, int N, int K, int head_dim, size_t* code_bytes,
                                 size_t* scale_bytes) {
  if (!code_bytes || !scale_bytes) return fail(I4D_ERR_NULL, "output pointer is NULL");
  i4d_status st = check_pack_args(kind, N, K, head_dim);
  if (st) return st;
  const int Np = packed_rows(kind, N);
  *code_bytes = (size_t)Np * (size_t)K;
  *scale_bytes = packed_scale_elems(Np, K) * sizeof(uint16_t);
  return ok();
}

i4d_status i4d_pack_weights_e4m3(i4d_proj_kind kind, const float* W0, const float* W1, const float* gamma,
                                 int N, int K, int head_dim, void* codes_out, uint16_t* scales_out,
                                 int threads) {
  return pack_e4m3_atoms(kind, W0, W1, gamma, N, K, head_dim, codes_out, scales_out, threads, quantize_group_e4m3);
}

i4d_status i4d_packed_sizes_mx(i4d_proj_kind kind, int N, int K, int head_dim, size_t* code_bytes,
                               size_t* scale_bytes) {
  if (!code_bytes || !scale_bytes) return fail(I4D_ERR_NULL, "output pointer is NULL");
  i4d_status st = check_pack_args(kind, N, K, head_dim);
  if (st) return st;
  const int Np = packed_rows(kind, N);
  *code_bytes = (size_t)Np * (size_t)K;
  *scale_bytes = packed_scale_elems(Np, K);
  return ok();
}

i4d_status i4d_pack_weights_mx(i4d_proj_kind kind, const float* W0, const float* W1, const float* gamma, int N,
                               int K, int head_dim, void* codes_out, uint8_t* scales_out, int threads) {
  return pack_e4m3_atoms(kind, W0, W1, gamma, N, K, head_dim, codes_out, scales_out, threads, quantize_group_mx);
}

i4d_status i4d_unpack_weights_mx(i4d_proj_kind kind, const void* codes, const uint8_t* scales, int N, int K,
                                 int head_dim, uint8_t* q_out, uint8_t* s_out) {
  return unpack_e4m3_atoms(kind, codes, scales, N, K, head_dim, q_out, s_out);
}

i4d_status i4d_unpack_weights_e4m3(i4d_proj_kind kind, const void* codes, const uint16_t* scales, int N, int K,
                                   int head_dim, uint8_t* q_out, uint16_t* s_out) {
  return unpack_e4m3_atoms(kind, codes, scales, N, K, head_dim, q_out, s_out);
}

i4d_status i4d_unpack_weights(i4d_proj_kind kind, const void* codes, const uint16_t* scales, int N,
                              int K, int head_dim, int8_t* q_out, uint16_t* s_out) {
  i4d_status st = check_pack_args(kind, N, K, head_dim);
  if (st) return st;
  if (!codes || !scales || !q_out || !s_out) return fail(I4D_ERR_NULL, "NULL pointer");
  const int Np = packed_rows(kind, N);
  const int G = groups_of(K);
  const uint8_t* c = (const uint8_t*)codes;
  for (int p = 0; p < Np; ++p) {
    int mat, row;
    source_row(kind, p, head_dim, &mat, &row);
    int out_row = mat * N + row;
    for (int k = 0; k < K; ++k) {
      int hi;
      size_t off = code_byte_offset(p, k, K, &hi);
      int u = hi ? (c[off] >> 4) : (c[off] & 15);
      q_out[(size_t)out_row * K + k] = (int8_t)(u - 8);
    }
    for (int g = 0; g < G; ++g) s_out[(size_t)out_row * G + g] = scales[scale_index(p, g, K)];
  }
  return ok();
}

i4d_status i4d_pack_lm_head(const float* W, const float* gamma, int V, int d, uint16_t* out_bf16,
                            int threads) {
  if (!W || !out_bf16) return fail(I4D_ERR_NULL, "W/out NULL");
  if (V <= 0 || d <= 0 || V % kStrip || d % kGroup)
    return fail(I4D_ERR_SHAPE, "LM head V=%d must be a multiple of 16, d=%d of 128", V, d);
  // tiles of 16 rows x 32 k ([V/16][d/32][16][32], 1 KiB each), so that
  // one 16-byte load per lane of the kernel's MFMA operand reads one
  // contiguous KiB
  parallel_for(V, threads, [&](long v0, long v1) {
    for (long v = v0; v < v1; ++v)
      for (int k = 0; k < d; ++k) {
        float w = W[(size_t)v * d + k];
        const size_t o = (((size_t)(v / kStrip) * (d / 32) + k / 32) * kStrip + v % kStrip) * 32 + k % 32;
        out_bf16[o] = f32_to_bf16_rne(gamma ? gamma[k] * w : w);
      }
  });
  return ok();
}

i4d_status i4d_kv_cache_bytes(int n_kv_heads, int head_dim, int64_t total_capacity,
                              size_t* k_code_bytes, size_t* v_code_bytes, size_t* k_scale_bytes,
                              size_t* v_scale_bytes) {
  if (!k_code_bytes || !v_code_bytes || !k_scale_bytes || !v_scale_bytes)
    return fail(I4D_ERR_NULL, "output pointer NULL");
  if (head_dim != 64 && head_dim != 128) return fail(I4D_ERR_UNSUPPORTED, "head_dim %d", head_dim);
  if (n_kv_heads <= 0 || total_capacity < 0 || total_capacity % kVBlock)
    return fail(I4D_ERR_SHAPE, "capacity %lld must be a non-negative multiple of 32",
                (long long)total_capacity);
  size_t slots = (size_t)total_capacity * n_kv_heads;
  *k_code_bytes = *v_code_bytes = slots * head_dim / 2;
  *k_scale_bytes = *v_scale_bytes = slots * sizeof(uint16_t);
  return ok();
}

i4d_status i4d_kv_unpack_host(const i4d_kv_cache* hc, const int64_t* row_base_host, int row,
                              int t0, int t1, int8_t* k_out, int8_t* v_out, uint16_t* ks_out,
                              uint16_t* vs_out) {
  if (!hc || !row_base_host || !k_out || !v_out || !ks_out || !vs_out)
    return fail(I4D_ERR_NULL, "NULL pointer");
  if (row < 0 || row >= hc->n_rows) return fail(I4D_ERR_RANGE, "row %d out of range", row);
  const int hd = hc->head_dim, nkv = hc->n_kv_heads;
  const int64_t base = row_base_host[row], cap = row_base_host[row + 1] - base;
  if (t0 < 0 || t1 > cap || t0 > t1) return fail(I4D_ERR_RANGE, "token range out of capacity");
  const uint8_t* kc = (const uint8_t*)hc->k_codes;
  const uint32_t* vc = (const uint32_t*)hc->v_codes;
  for (int t = t0; t < t1; ++t)
    for (int j = 0; j < nkv; ++j) {
      int64_t region = base * nkv + (int64_t)j * cap;  // first slot of (row, head)
      int64_t slot = region + t;
      size_t o = (size_t)(t - t0) * nkv + j;
      ks_out[o] = hc->k_scales[slot];
      vs_out[o] = hc->v_scales[slot];
      for (int c = 0; c < hd; ++c) {
        int hi;
        int b = key_byte_in_slot(c, hd, &hi);
        uint8_t byte = kc[(size_t)slot * (hd / 2) + b];
        k_out[o * hd + c] = (int8_t)((hi ? byte >> 4 : byte & 15) - 8);
        int ns;
        int dw = value_dword_in_block(t % kVBlock, c, hd, &ns);
        size_t blk = (size_t)(region / kVBlock + t / kVBlock);
        uint32_t word = vc[blk * 4 * hd + dw];
        v_out[o * hd + c] = (int8_t)(((word >> (4 * ns)) & 15) - 8);
      }
    }
  return ok();
}

i4d_status i4d_attention_workspace_bytes(const i4d_layer_shape* shape, int M, int max_ctx_len,
                                         int num_splits, size_t* bytes) {
  i4d_status st = check_shape(shape);
  if (st) return st;
  if (!bytes) return fail(I4D_ERR_NULL, "bytes NULL");
  if (M < 1 || M > I4D_MAX_ROWS) return fail(I4D_ERR_RANGE, "M=%d outside [1, 32]", M);
  if (max_ctx_len < 1) return fail(I4D_ERR_RANGE, "max_ctx_len must be >= 1");
  if (num_splits < 0 || num_splits > I4D_MAX_SPLITS)
    return fail(I4D_ERR_RANGE, "num_splits %d outside [0, %d]", num_splits, I4D_MAX_SPLITS);
  const int S = attn_plan(shape, M, max_ctx_len, num_splits).S;
  *bytes = attn_ws_layout(shape, M, S).total;
  return ok();
}

i4d_status i4d_workspace_layout_of(const i4d_layer_shape* s, int M, int max_ctx_len,
                                   int num_splits, i4d_workspace_layout* out) {
  if (!out) return fail(I4D_ERR_NULL, "layout NULL");
  size_t attn_bytes;
  i4d_status st = i4d_attention_workspace_bytes(s, M, max_ctx_len, num_splits, &attn_bytes);
  if (st) return st;
  if (M == 1)  // the one-launch step may use another split count, and adds its flagged words
    attn_bytes = std::max(attn_bytes, attn_ws_layout(s, 1, step_m1_splits(s, max_ctx_len, num_splits)).total +
                                          step_ll_layout(s).total);
  size_t nq = (size_t)M * s->n_q_heads * s->head_dim;
  size_t nk = (size_t)M * s->n_kv_heads * s->head_dim;
  // the four projections run one after another and leave their counters
  // at zero, so they share one split buffer
  const int nqkv = (s->n_q_heads + 2 * s->n_kv_heads) * s->head_dim;
  const SplitNeed need[4] = {projection_split_need(nqkv, s->d_model, M),
                             projection_split_need(s->d_model, s->n_q_heads * s->head_dim, M),
                             projection_split_need(2 * s->d_ffn, s->d_model, M),
                             projection_split_need(s->d_model, s->d_ffn, M)};
  size_t cnt = 0, part = 0;
  for (const SplitNeed& n : need) {
    cnt = std::max(cnt, n.counters);
    part = std::max(part, n.part_bytes);
  }
  if (cnt * sizeof(unsigned) > kSplitCntBytes)
    return fail(I4D_ERR_UNSUPPORTED, "K split needs %zu arrival counters (at most %zu)", cnt,
                kSplitCntBytes / sizeof(unsigned));
  // counters first, at fixed offsets (see kSplitCntBytes); the split
  // partial tiles last
  size_t off = 0;
  out->sync = off;       off += align256(kStepSyncBytes);
  out->split_cnt = off;  off += align256(kSplitCntBytes);
  out->q = off;       off += align256(nq * 4);
  out->k = off;       off += align256(nk * 2);
  out->v = off;       off += align256(nk * 2);
  out->attn = off;    off += align256(nq * 2);
  out->h = off;       off += align256((size_t)M * s->d_model * 4);
  out->h_bf16 = off;  off += align256((size_t)M * s->d_model * 2);
  out->a = off;       off += align256((size_t)M * s->d_ffn * 2);
  out->attn_ws = off; off += align256(attn_bytes);
  out->split_part = off; off += align256(part);
  out->total = off;
  return ok();
}

i4d_status i4d_workspace_bytes(const i4d_layer_shape* shape, int M, int max_ctx_len,
                               int num_splits, size_t* bytes) {
  if (!bytes) return fail(I4D_ERR_NULL, "bytes NULL");
  i4d_workspace_layout l;
  i4d_status st = i4d_workspace_layout_of(shape, M, max_ctx_len, num_splits, &l);
  if (st) return st;
  *bytes = l.total;
  return ok();
}

i4d_status i4d_lm_head_workspace_bytes(int V, int M, size_t* bytes) {
  if (!bytes) return fail(I4D_ERR_NULL, "bytes NULL");
  if (V <= 0 || V % kStrip) return fail(I4D_ERR_SHAPE, "V=%d must be a multiple of 16", V);
  if (M < 1 || M > I4D_MAX_ROWS) return fail(I4D_ERR_RANGE, "M=%d outside [1, 32]", M);
  *bytes = lm_ws_layout(V, M).total;
  return ok();
}

}  // extern "C"
