// attn.hip - stand-alone KV append, attention and split-combine kernels
// (gfx950); the device code lives in attn_core.h.
#include <math.h>

#include "attn.h"
#include "attn_core.h"
#include "device_common.h"

namespace i4d {

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
  append_vector<HD>(kv, src, base * kv.n_kv + (int64_t)head * cap, pos, kind, lane);
}

template <int HD, int NWA>
__global__ __launch_bounds__(NWA * 64) void attn_kernel(AttnArgs a) {
  __shared__ float lds[attn_lds_floats<HD, NWA>()];
  const int S = a.S;
  const int s = blockIdx.x % S;
  const int rest = blockIdx.x / S;
  attn_body<HD, NWA, false>(a, rest / a.kv.n_kv, rest % a.kv.n_kv, s, lds, [] {});
}

template <int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= a.M * a.n_q) return;
  float lsum, o0, o1;
  combine_head<HD>(a, (size_t)idx, lane, lsum, o0, o1);
  finish_head<HD>(a, (size_t)idx, lsum, o0, o1, lane);
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

template <int HD>
static void launch_attn_hd(const AttnArgs& a, int nwa, hipStream_t st) {
  const int grid = a.M * a.kv.n_kv * a.S;
  if (nwa == 4)
    hipLaunchKernelGGL((attn_kernel<HD, 4>), dim3(grid), dim3(4 * 64), 0, st, a);
  else
    hipLaunchKernelGGL((attn_kernel<HD, 8>), dim3(grid), dim3(8 * 64), 0, st, a);
}

i4d_status launch_attention(const AttnArgs& a, int nwa, bool combine, hipStream_t st) {
  if (nwa != 4 && nwa != 8) return fail(I4D_ERR_RANGE, "attention waves %d", nwa);
  if (a.G < 1 || a.G > 8) return fail(I4D_ERR_UNSUPPORTED, "GQA group %d > 8", a.G);
  if (a.kv.hd == 128)
    launch_attn_hd<128>(a, nwa, st);
  else
    launch_attn_hd<64>(a, nwa, st);
  if (combine && a.S > 1) {
    const dim3 grid((a.M * a.n_q + 3) / 4);
    if (a.kv.hd == 128)
      hipLaunchKernelGGL(attn_combine_kernel<128>, grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(attn_combine_kernel<64>, grid, dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(I4D_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace i4d
