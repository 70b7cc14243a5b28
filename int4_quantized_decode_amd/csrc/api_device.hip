// api_device.hip - C-ABI entry points that enqueue GPU work.  Every argument
// is validated on the host before the first launch; nothing is allocated and
// nothing synchronises.
#include <math.h>

#include "attn.h"
#include "device_common.h"
#include "i4d_internal.h"
#include "lmhead.h"
#include "proj.h"
#include "step.h"

using namespace i4d;

#define I4D_TRY(expr)                \
  do {                               \
    i4d_status st_ = (expr);         \
    if (st_ != I4D_OK) return st_;   \
  } while (0)

namespace i4d {

i4d_status need(const void* p, const char* what) {
  if (!p) return fail(I4D_ERR_NULL, "%s is NULL", what);
  if (!aligned16(p)) return fail(I4D_ERR_ALIGN, "%s is not 16-byte aligned", what);
  return ok();
}

}  // namespace i4d

namespace {

i4d_status check_rows(int M) {
  if (M < 1 || M > I4D_MAX_ROWS) return fail(I4D_ERR_RANGE, "M=%d outside [1, %d]", M, I4D_MAX_ROWS);
  return ok();
}

i4d_status check_layer(const i4d_layer* L) {
  if (!L) return fail(I4D_ERR_NULL, "layer is NULL");
  I4D_TRY(check_shape(&L->shape));
  I4D_TRY(need(L->qkv_codes, "qkv_codes"));
  I4D_TRY(need(L->qkv_scales, "qkv_scales"));
  I4D_TRY(need(L->o_codes, "o_codes"));
  I4D_TRY(need(L->o_scales, "o_scales"));
  I4D_TRY(need(L->gu_codes, "gu_codes"));
  I4D_TRY(need(L->gu_scales, "gu_scales"));
  I4D_TRY(need(L->down_codes, "down_codes"));
  I4D_TRY(need(L->down_scales, "down_scales"));
  return ok();
}

}  // namespace

namespace i4d {

i4d_status check_cache(const i4d_kv_cache* c, const i4d_layer_shape* s, int M) {
  if (!c) return fail(I4D_ERR_NULL, "cache is NULL");
  I4D_TRY(need(c->k_codes, "cache k_codes"));
  I4D_TRY(need(c->v_codes, "cache v_codes"));
  I4D_TRY(need(c->k_scales, "cache k_scales"));
  I4D_TRY(need(c->v_scales, "cache v_scales"));
  if (!c->row_base) return fail(I4D_ERR_NULL, "cache row_base is NULL");
  if (((uintptr_t)c->row_base & 7u) != 0) return fail(I4D_ERR_ALIGN, "row_base not 8-byte aligned");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(I4D_ERR_UNSUPPORTED, "cache head_dim %d", c->head_dim);
  if (c->n_kv_heads <= 0) return fail(I4D_ERR_SHAPE, "cache n_kv_heads %d", c->n_kv_heads);
  if (c->total_capacity <= 0 || c->total_capacity % kVBlock)
    return fail(I4D_ERR_SHAPE, "cache capacity %lld must be a positive multiple of 32",
                (long long)c->total_capacity);
  if (s && (c->head_dim != s->head_dim || c->n_kv_heads != s->n_kv_heads))
    return fail(I4D_ERR_SHAPE, "cache (n_kv %d, hd %d) does not match the layer (n_kv %d, hd %d)",
                c->n_kv_heads, c->head_dim, s->n_kv_heads, s->head_dim);
  if (M > c->n_rows) return fail(I4D_ERR_SHAPE, "M=%d exceeds cache rows %d", M, c->n_rows);
  return ok();
}

KvArgs kv_args(const i4d_kv_cache* c) {
  KvArgs k;
  k.k_codes = (uint8_t*)c->k_codes;
  k.v_codes = (uint32_t*)c->v_codes;
  k.k_scales = c->k_scales;
  k.v_scales = c->v_scales;
  k.row_base = c->row_base;
  k.n_rows = c->n_rows;
  k.n_kv = c->n_kv_heads;
  k.hd = c->head_dim;
  k.err_word = c->err_word;
  return k;
}

}  // namespace i4d

namespace {

ProjArgs proj_args(const void* codes, const uint16_t* scales, const uint16_t* x, int Np, int K,
                   int M, float eps) {
  ProjArgs a = {};
  a.codes = (const uint8_t*)codes;
  a.scales = scales;
  a.x = x;
  a.Np = Np;
  a.K = K;
  a.G = groups_of(K);
  a.G8 = g8_of(K);
  a.M = M;
  a.eps = eps;
  return a;
}

ProjArgs qkv_args(const i4d_layer* L, const uint16_t* x, const int32_t* ctx_len, int M, float* q,
                  uint16_t* k, uint16_t* v) {
  const i4d_layer_shape& s = L->shape;
  ProjArgs a = proj_args(L->qkv_codes, L->qkv_scales, x,
                         (s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim, s.d_model, M, s.rms_eps);
  a.q_out = q;
  a.k_out = k;
  a.v_out = v;
  a.ctx_len = ctx_len;
  a.n_q = s.n_q_heads;
  a.n_kv = s.n_kv_heads;
  a.hd = s.head_dim;
  a.theta = s.rope_theta;
  a.rope_ratio = pow((double)s.rope_theta, -2.0 / (double)s.head_dim);
  return a;
}

i4d_status do_qkv(const i4d_layer* L, const uint16_t* x, const int32_t* ctx_len, int M, float* q,
                  uint16_t* k, uint16_t* v, hipStream_t st) {
  return launch_projection(EPI_QKV, qkv_args(L, x, ctx_len, M, q, k, v), st);
}

AttnArgs attention_args(const i4d_kv_cache* c, const i4d_layer_shape& s, const float* q,
                        const int32_t* ctx_len, int M, int max_ctx_len, int S, void* ws, float* attn_f32,
                        uint16_t* attn_bf16, const uint16_t* k_new, const uint16_t* v_new) {
  AttnArgs a = {};
  a.kv = kv_args(c);
  a.q = q;
  a.ctx_len = ctx_len;
  a.k_new = k_new;
  a.v_new = v_new;
  a.M = M;
  a.n_q = s.n_q_heads;
  a.G = s.n_q_heads / s.n_kv_heads;
  a.S = S;
  a.bps = std::max(1, ((max_ctx_len + kVBlock - 1) / kVBlock + S - 1) / S);
  a.score_scale = (float)(1.4426950408889634 / ((double)s.head_dim * sqrt((double)s.head_dim)));
  AttnWs w = attn_ws_layout(&s, M, a.S);
  a.part_ml = (float*)((char*)ws + w.ml);
  a.part_o = (float*)((char*)ws + w.o);
  a.attn_f32 = attn_f32;
  a.attn_bf16 = attn_bf16;
  return a;
}

i4d_status do_attention(const i4d_kv_cache* c, const i4d_layer_shape& s, const float* q,
                        const int32_t* ctx_len, int M, int max_ctx_len, int num_splits, void* ws,
                        float* attn_f32, uint16_t* attn_bf16, const uint16_t* k_new,
                        const uint16_t* v_new, bool combine, hipStream_t st) {
  const AttnPlan plan = attn_plan(&s, M, max_ctx_len, num_splits);
  const AttnArgs a = attention_args(c, s, q, ctx_len, M, max_ctx_len, plan.S, ws, attn_f32, attn_bf16, k_new, v_new);
  return launch_attention(a, plan.nwa, combine, st);
}

ProjArgs o_args(const i4d_layer* L, const uint16_t* attn, const uint16_t* x, int M, float* h,
                uint16_t* hb) {
  const i4d_layer_shape& s = L->shape;
  ProjArgs a = proj_args(L->o_codes, L->o_scales, attn, s.d_model, s.n_q_heads * s.head_dim, M,
                         s.rms_eps);
  a.resid_bf16 = x;
  a.h_f32 = h;
  a.h_bf16 = hb;
  return a;
}

ProjArgs gu_args(const i4d_layer* L, const uint16_t* hb, int M, uint16_t* out) {
  const i4d_layer_shape& s = L->shape;
  ProjArgs a = proj_args(L->gu_codes, L->gu_scales, hb, 2 * s.d_ffn, s.d_model, M, s.rms_eps);
  a.a_out = out;
  return a;
}

ProjArgs down_args(const i4d_layer* L, const uint16_t* act, const float* h, int M, uint16_t* out) {
  const i4d_layer_shape& s = L->shape;
  ProjArgs a = proj_args(L->down_codes, L->down_scales, act, s.d_model, s.d_ffn, M, s.rms_eps);
  a.resid_f32 = h;
  a.out_bf16 = out;
  return a;
}

i4d_status do_o(const i4d_layer* L, const uint16_t* attn, const uint16_t* x, int M, float* h,
                uint16_t* hb, hipStream_t st) {
  return launch_projection(EPI_O, o_args(L, attn, x, M, h, hb), st);
}

i4d_status do_gu(const i4d_layer* L, const uint16_t* hb, int M, uint16_t* out, hipStream_t st) {
  return launch_projection(EPI_GU, gu_args(L, hb, M, out), st);
}

i4d_status do_down(const i4d_layer* L, const uint16_t* act, const float* h, int M, uint16_t* out,
                   hipStream_t st) {
  return launch_projection(EPI_DOWN, down_args(L, act, h, M, out), st);
}

__global__ void zero_fill_kernel(u32x4_t* p, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = u32x4_t{0u, 0u, 0u, 0u};
}

}  // namespace

namespace i4d {

i4d_status check_decode_step(const i4d_layer* layer, const i4d_kv_cache* cache, const uint16_t* x_in,
                             const uint16_t* x_out, const int32_t* ctx_len, int M, int max_ctx_len,
                             int num_splits, const float* attn_f32, i4d_workspace_layout* wl) {
  I4D_TRY(check_layer(layer));
  I4D_TRY(check_rows(M));
  I4D_TRY(check_cache(cache, &layer->shape, M));
  I4D_TRY(need(x_in, "x_in"));
  I4D_TRY(need(x_out, "x_out"));
  I4D_TRY(need(ctx_len, "ctx_len"));
  if (attn_f32 && !aligned16(attn_f32)) return fail(I4D_ERR_ALIGN, "attn_f32 not 16-byte aligned");
  if (x_in == x_out) return fail(I4D_ERR_RANGE, "x_in and x_out must not alias");
  if (max_ctx_len < 1 || max_ctx_len > cache->total_capacity)
    return fail(I4D_ERR_RANGE, "max_ctx_len %d outside [1, capacity]", max_ctx_len);
  return i4d_workspace_layout_of(&layer->shape, M, max_ctx_len, num_splits, wl);
}

i4d_status run_decode_step(const i4d_layer* layer, const i4d_kv_cache* cache, const uint16_t* x_in,
                           uint16_t* x_out, const int32_t* ctx_len, int M, int max_ctx_len, int num_splits,
                           char* ws, const i4d_workspace_layout& wl, size_t split_part_bytes, float* attn_f32,
                           hipStream_t st, int fmt, uint64_t* stamps) {
  float* q = (float*)(ws + wl.q);
  uint16_t* k = (uint16_t*)(ws + wl.k);
  uint16_t* v = (uint16_t*)(ws + wl.v);
  uint16_t* attn = (uint16_t*)(ws + wl.attn);
  float* h = (float*)(ws + wl.h);
  uint16_t* hb = (uint16_t*)(ws + wl.h_bf16);
  uint16_t* act = (uint16_t*)(ws + wl.a);
  const i4d_layer_shape& s = layer->shape;

  if (fmt == kFmtInt4 && M == 1 && step_m1_supported(&s)) {
    StepInputs in;
    in.layer = layer;
    in.qkv = qkv_args(layer, x_in, ctx_len, 1, q, k, v);
    in.o = o_args(layer, attn, x_in, 1, h, hb);
    in.gu = gu_args(layer, hb, 1, act);
    in.down = down_args(layer, act, h, 1, x_out);
    const int S1 = step_m1_splits(&s, max_ctx_len, num_splits);
    in.attn = attention_args(cache, s, q, ctx_len, 1, max_ctx_len, S1, ws + wl.attn_ws, attn_f32, attn, k, v);
    // the flagged exchange words follow the attention partials
    char* llb = ws + wl.attn_ws + attn_ws_layout(&s, 1, S1).total;
    const StepLl ll = step_ll_layout(&s);
    in.qkv.q_ll = (uint64_t*)(llb + ll.q);
    in.qkv.k_ll = (uint64_t*)(llb + ll.k);
    in.qkv.v_ll = (uint64_t*)(llb + ll.v);
    in.attn.q_ll = in.qkv.q_ll;
    in.attn.k_ll = in.qkv.k_ll;
    in.attn.v_ll = in.qkv.v_ll;
    in.sync = (unsigned*)(ws + wl.sync);
    in.stamps = stamps;
    return launch_step_m1(in, st);
  }
  // the projections may split K across workgroups through the workspace
  // (INT4); the weights' format selects the kernels
  auto split = [&](ProjArgs a) {
    a.split_cnt = (unsigned*)(ws + wl.split_cnt);
    a.split_part = (float*)(ws + wl.split_part);
    a.split_bytes = split_part_bytes;
    a.fmt = fmt;
    return a;
  };
  I4D_TRY(launch_projection(EPI_QKV, split(qkv_args(layer, x_in, ctx_len, M, q, k, v)), st));
  // the attention launch first appends the new token of row m at position
  // ctx_len[m] - 1 of cache row m (inside the workgroup that owns that block)
  I4D_TRY(do_attention(cache, s, q, ctx_len, M, max_ctx_len, num_splits, ws + wl.attn_ws, attn_f32,
                       attn, k, v, true, st));
  I4D_TRY(launch_projection(EPI_O, split(o_args(layer, attn, x_in, M, h, hb)), st));
  I4D_TRY(launch_projection(EPI_GU, split(gu_args(layer, hb, M, act)), st));
  I4D_TRY(launch_projection(EPI_DOWN, split(down_args(layer, act, h, M, x_out)), st));
  return ok();
}

i4d_status launch_zero_fill(void* p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return ok();
  const size_t n16 = bytes / 16;
  const unsigned grid = (unsigned)std::min<size_t>(1024, (n16 + 255) / 256);
  hipLaunchKernelGGL(zero_fill_kernel, dim3(grid), dim3(256), 0, st, (u32x4_t*)p, n16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(I4D_ERR_HIP, "zero fill: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace i4d

extern "C" {

i4d_status i4d_attn_qkv(const i4d_layer* layer, const uint16_t* x, const int32_t* ctx_len, int M,
                        float* q_out, uint16_t* k_out, uint16_t* v_out, void* stream) {
  I4D_TRY(check_layer(layer));
  I4D_TRY(check_rows(M));
  I4D_TRY(need(x, "x"));
  I4D_TRY(need(ctx_len, "ctx_len"));
  I4D_TRY(need(q_out, "q_out"));
  I4D_TRY(need(k_out, "k_out"));
  I4D_TRY(need(v_out, "v_out"));
  return do_qkv(layer, x, ctx_len, M, q_out, k_out, v_out, (hipStream_t)stream);
}

i4d_status i4d_kv_append(const i4d_kv_cache* cache, const uint16_t* k, const uint16_t* v,
                         const int32_t* row_idx, const int32_t* pos, int T, void* stream) {
  I4D_TRY(check_cache(cache, nullptr, 0));
  if (T < 0) return fail(I4D_ERR_RANGE, "T=%d must be >= 0", T);
  if (T == 0) return ok();
  I4D_TRY(need(k, "k"));
  I4D_TRY(need(v, "v"));
  I4D_TRY(need(pos, "pos"));
  if (row_idx && !aligned16(row_idx)) return fail(I4D_ERR_ALIGN, "row_idx not 16-byte aligned");
  if (!row_idx && T > cache->n_rows)
    return fail(I4D_ERR_SHAPE, "T=%d tokens without row_idx need T <= n_rows (%d)", T, cache->n_rows);
  AppendArgs a;
  a.kv = kv_args(cache);
  a.k = k;
  a.v = v;
  a.row_idx = row_idx;
  a.pos = pos;
  a.len = nullptr;
  a.T = T;
  return launch_kv_append(a, (hipStream_t)stream);
}

i4d_status i4d_attention(const i4d_kv_cache* cache, const i4d_layer_shape* shape, const float* q,
                         const int32_t* ctx_len, int M, int max_ctx_len, int num_splits,
                         void* workspace, size_t workspace_bytes, float* attn_f32,
                         uint16_t* attn_bf16, void* stream) {
  I4D_TRY(check_shape(shape));
  I4D_TRY(check_rows(M));
  I4D_TRY(check_cache(cache, shape, M));
  I4D_TRY(need(q, "q"));
  I4D_TRY(need(ctx_len, "ctx_len"));
  I4D_TRY(need(attn_bf16, "attn_bf16"));
  I4D_TRY(need(workspace, "workspace"));
  if (attn_f32 && !aligned16(attn_f32)) return fail(I4D_ERR_ALIGN, "attn_f32 not 16-byte aligned");
  if (max_ctx_len < 1 || max_ctx_len > cache->total_capacity)
    return fail(I4D_ERR_RANGE, "max_ctx_len %d outside [1, capacity]", max_ctx_len);
  size_t need_ws;
  I4D_TRY(i4d_attention_workspace_bytes(shape, M, max_ctx_len, num_splits, &need_ws));
  if (workspace_bytes < need_ws)
    return fail(I4D_ERR_WORKSPACE, "attention workspace %zu < %zu bytes", workspace_bytes, need_ws);
  return do_attention(cache, *shape, q, ctx_len, M, max_ctx_len, num_splits, workspace, attn_f32,
                      attn_bf16, nullptr, nullptr, true, (hipStream_t)stream);
}

i4d_status i4d_attn_out_proj(const i4d_layer* layer, const uint16_t* attn_bf16, const uint16_t* x,
                             int M, float* h_f32, uint16_t* h_bf16, void* stream) {
  I4D_TRY(check_layer(layer));
  I4D_TRY(check_rows(M));
  I4D_TRY(need(attn_bf16, "attn_bf16"));
  I4D_TRY(need(x, "x"));
  I4D_TRY(need(h_f32, "h_f32"));
  I4D_TRY(need(h_bf16, "h_bf16"));
  return do_o(layer, attn_bf16, x, M, h_f32, h_bf16, (hipStream_t)stream);
}

i4d_status i4d_ffn_gate_up(const i4d_layer* layer, const uint16_t* h_bf16, int M, uint16_t* a_out,
                           void* stream) {
  I4D_TRY(check_layer(layer));
  I4D_TRY(check_rows(M));
  I4D_TRY(need(h_bf16, "h_bf16"));
  I4D_TRY(need(a_out, "a_out"));
  return do_gu(layer, h_bf16, M, a_out, (hipStream_t)stream);
}

i4d_status i4d_ffn_down(const i4d_layer* layer, const uint16_t* a, const float* h, int M,
                        uint16_t* x_out, void* stream) {
  I4D_TRY(check_layer(layer));
  I4D_TRY(check_rows(M));
  I4D_TRY(need(a, "a"));
  I4D_TRY(need(h, "h"));
  I4D_TRY(need(x_out, "x_out"));
  return do_down(layer, a, h, M, x_out, (hipStream_t)stream);
}

i4d_status i4d_decode_block_step(const i4d_layer* layer, const i4d_kv_cache* cache,
                                 const uint16_t* x_in, uint16_t* x_out, const int32_t* ctx_len,
                                 int M, int max_ctx_len, int num_splits, void* workspace,
                                 size_t workspace_bytes, float* attn_f32, void* stream) {
  i4d_workspace_layout wl;
  I4D_TRY(check_decode_step(layer, cache, x_in, x_out, ctx_len, M, max_ctx_len, num_splits, attn_f32, &wl));
  I4D_TRY(need(workspace, "workspace"));
  if (workspace_bytes < wl.total)
    return fail(I4D_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, wl.total);
  return run_decode_step(layer, cache, x_in, x_out, ctx_len, M, max_ctx_len, num_splits, (char*)workspace, wl,
                         wl.total - wl.split_part, attn_f32, (hipStream_t)stream, kFmtInt4);
}

i4d_status i4d_decode_block_step_timeline(const i4d_layer* layer, const i4d_kv_cache* cache, const uint16_t* x_in,
                                          uint16_t* x_out, const int32_t* ctx_len, int M, int max_ctx_len,
                                          int num_splits, void* workspace, size_t workspace_bytes, float* attn_f32,
                                          uint64_t* stamps, size_t stamps_count, void* stream) {
  i4d_workspace_layout wl;
  I4D_TRY(check_decode_step(layer, cache, x_in, x_out, ctx_len, M, max_ctx_len, num_splits, attn_f32, &wl));
  I4D_TRY(need(workspace, "workspace"));
  if (workspace_bytes < wl.total)
    return fail(I4D_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, wl.total);
  if (M != 1 || !step_m1_supported(&layer->shape))
    return fail(I4D_ERR_UNSUPPORTED, "the timeline covers the one-launch step (M = 1, a shape it supports)");
  I4D_TRY(need(stamps, "stamps"));
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(I4D_ERR_HIP, "device query failed");
  if (stamps_count < (size_t)cus * I4D_STEP_STAMPS)
    return fail(I4D_ERR_RANGE, "stamps holds %zu values, the step needs %d x %d", stamps_count, cus,
                I4D_STEP_STAMPS);
  return run_decode_step(layer, cache, x_in, x_out, ctx_len, M, max_ctx_len, num_splits, (char*)workspace, wl,
                         wl.total - wl.split_part, attn_f32, (hipStream_t)stream, kFmtInt4, stamps);
}

i4d_status i4d_decode_block_step_e4m3(const i4d_layer* layer, const i4d_kv_cache* cache, const uint16_t* x_in,
                                      uint16_t* x_out, const int32_t* ctx_len, int M, int max_ctx_len,
                                      int num_splits, void* workspace, size_t workspace_bytes, float* attn_f32,
                                      void* stream) {
  i4d_workspace_layout wl;
  I4D_TRY(check_decode_step(layer, cache, x_in, x_out, ctx_len, M, max_ctx_len, num_splits, attn_f32, &wl));
  I4D_TRY(need(workspace, "workspace"));
  if (workspace_bytes < wl.total)
    return fail(I4D_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, wl.total);
  return run_decode_step(layer, cache, x_in, x_out, ctx_len, M, max_ctx_len, num_splits, (char*)workspace, wl,
                         wl.total - wl.split_part, attn_f32, (hipStream_t)stream, kFmtE4M3);
}

i4d_status i4d_attn_out_proj_e4m3(const i4d_layer* layer, const uint16_t* attn_bf16, const uint16_t* x, int M,
                                  float* h_f32, uint16_t* h_bf16, void* stream) {
  I4D_TRY(check_layer(layer));
  I4D_TRY(check_rows(M));
  I4D_TRY(need(attn_bf16, "attn_bf16"));
  I4D_TRY(need(x, "x"));
  I4D_TRY(need(h_f32, "h_f32"));
  I4D_TRY(need(h_bf16, "h_bf16"));
  ProjArgs a = o_args(layer, attn_bf16, x, M, h_f32, h_bf16);
  a.fmt = kFmtE4M3;
  return launch_projection(EPI_O, a, (hipStream_t)stream);
}

i4d_status i4d_projection_plan_of(const i4d_layer_shape* shape, int stage, int M, i4d_projection_plan* out) {
  I4D_TRY(check_shape(shape));
  I4D_TRY(check_rows(M));
  if (!out) return fail(I4D_ERR_NULL, "out is NULL");
  if (stage < 0 || stage > 3) return fail(I4D_ERR_RANGE, "stage %d outside [0, 3]", stage);
  i4d_workspace_layout wl;
  I4D_TRY(i4d_workspace_layout_of(shape, M, 1, 0, &wl));
  // the arguments as the block step builds them: null data pointers (only
  // the plan is computed) and the workspace's split buffer, whose pointers
  // only have to be non-null for the plan to consider a split of K
  const i4d_layer_shape& s = *shape;
  i4d_layer L = {};
  L.shape = s;
  ProjArgs a;
  int epi = EPI_QKV;
  switch (stage) {
    case 0: a = qkv_args(&L, nullptr, nullptr, M, nullptr, nullptr, nullptr); epi = EPI_QKV; break;
    case 1: a = o_args(&L, nullptr, nullptr, M, nullptr, nullptr); epi = EPI_O; break;
    case 2: a = gu_args(&L, nullptr, M, nullptr); epi = EPI_GU; break;
    default: a = down_args(&L, nullptr, nullptr, M, nullptr); epi = EPI_DOWN; break;
  }
  if (M > 1) {
    a.split_cnt = reinterpret_cast<unsigned*>(wl.split_cnt + 256);
    a.split_part = reinterpret_cast<float*>(wl.split_part + 256);
    a.split_bytes = wl.total - wl.split_part;
  }
  return projection_plan_of(epi, a, out);
}

i4d_status i4d_decode_step_is_one_launch(const i4d_layer_shape* shape, int M, int* one_launch) {
  I4D_TRY(check_shape(shape));
  if (!one_launch) return fail(I4D_ERR_NULL, "one_launch is NULL");
  *one_launch = (M == 1 && step_m1_supported(shape)) ? 1 : 0;
  return ok();
}

i4d_status i4d_workspace_init(void* workspace, size_t bytes, void* stream) {
  I4D_TRY(need(workspace, "workspace"));
  if (bytes % 16) return fail(I4D_ERR_RANGE, "workspace bytes %zu not a multiple of 16", bytes);
  return launch_zero_fill(workspace, bytes, (hipStream_t)stream);
}

i4d_status i4d_lm_head_argmax(const uint16_t* w_lm, int V, int d, const uint16_t* h, int M,
                              float rms_eps, float* logits_out, int32_t* token_out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  I4D_TRY(check_rows(M));
  I4D_TRY(need(w_lm, "w_lm"));
  I4D_TRY(need(h, "h"));
  I4D_TRY(need(token_out, "token_out"));
  I4D_TRY(need(workspace, "workspace"));
  if (logits_out && !aligned16(logits_out)) return fail(I4D_ERR_ALIGN, "logits not aligned");
  if (V <= 0 || V % kStrip || d <= 0 || d % kGroup)
    return fail(I4D_ERR_SHAPE, "LM head V=%d (multiple of 16), d=%d (multiple of 128)", V, d);
  if (!(rms_eps > 0.f)) return fail(I4D_ERR_RANGE, "rms_eps must be > 0");
  size_t need_ws;
  I4D_TRY(i4d_lm_head_workspace_bytes(V, M, &need_ws));
  if (workspace_bytes < need_ws)
    return fail(I4D_ERR_WORKSPACE, "LM head workspace %zu < %zu", workspace_bytes, need_ws);
  LmWs w = lm_ws_layout(V, M);
  LmArgs a;
  a.w = w_lm;
  a.h = h;
  a.V = V;
  a.d = d;
  a.M = M;
  a.nwaves = w.nwaves;
  a.eps = rms_eps;
  a.logits = logits_out;
  a.part_val = (float*)((char*)workspace + w.val);
  a.part_idx = (int32_t*)((char*)workspace + w.idx);
  a.token = token_out;
  return launch_lm_head(a, (hipStream_t)stream);
}

}  // extern "C"
