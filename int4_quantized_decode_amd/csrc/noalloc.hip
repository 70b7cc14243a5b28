// noalloc.hip - the decode step for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that
// forbid hipMalloc): i4d_decode_block_step with its workspace in a
// library-owned device array instead of a caller's buffer.
//
// `scratch` is one file-scope device array per GPU (every device that loads
// the library holds its own copy until the process ends).  Host code never
// passes the array's name to a kernel or a copy: its device address is
// looked up once per device with hipGetSymbolAddress and kept.
//
// Layout of the array: the step's workspace layout (i4d_workspace_layout_of),
// whose counters sit at fixed offsets at its start (the one-launch step's
// sync region, then the projections' K-split arrival counters) whatever
// the shape and M of a call, with the other intermediates after them.
// Every completed step leaves its counters ready for the next call, so a
// call never sees another call's stale counters; the intermediates are
// written before they are read.  The array is cleared once, at the first
// call on a device.
// Calls that overlap on one GPU (two streams, or two threads) race on the
// array.
#include <mutex>

#include "device_common.h"
#include "i4d_internal.h"
#include "proj.h"
#include "step.h"

namespace i4d {
namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;         // I4D_NOALLOC_SCRATCH_BYTES

static_assert(kScratchBytes == I4D_NOALLOC_SCRATCH_BYTES, "header and library disagree on the scratch size");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];
bool g_cleared[kMaxDevices];

// the device address of this device's scratch (looked up on first use);
// `first` is set on the call that looked it up
i4d_status scratch_of(int dev, void** out, bool* first) {
  std::lock_guard<std::mutex> lock(g_mu);
  *first = false;
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(I4D_ERR_HIP, "scratch address of device %d: %s", dev, hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  if (!g_cleared[dev]) {
    g_cleared[dev] = true;
    *first = true;
  }
  *out = g_ptr[dev];
  return ok();
}

}  // namespace
}  // namespace i4d

using namespace i4d;

extern "C" i4d_status i4d_decode_block_step_noalloc(const i4d_layer* layer, const i4d_kv_cache* cache,
                                                    const uint16_t* x_in, uint16_t* x_out,
                                                    const int32_t* ctx_len, int M, int max_ctx_len,
                                                    int num_splits, float* attn_f32, void* stream) {
  i4d_workspace_layout wl;
  i4d_status st =
      check_decode_step(layer, cache, x_in, x_out, ctx_len, M, max_ctx_len, num_splits, attn_f32, &wl);
  if (st != I4D_OK) return st;
  // The scratch holds the step's workspace layout as it is: its counters
  // sit at the start (fixed offsets for every shape), so they keep their
  // places from one call to the next whatever the shapes.
  if (wl.total > kScratchBytes)
    return fail(I4D_ERR_WORKSPACE,
                "this step needs %zu bytes of scratch; the no-allocation entry point holds %zu: use "
                "i4d_decode_block_step with a workspace",
                wl.total, kScratchBytes);
  const size_t split_part_bytes = wl.total - wl.split_part;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(I4D_ERR_HIP, "no usable current device");
  void* base = nullptr;
  bool first = false;
  st = scratch_of(dev, &base, &first);
  if (st != I4D_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  // the counters start at zero on this device, and so do the one-launch
  // step's flagged exchange words (a fill kernel on the caller's stream,
  // ordered before the step)
  if (first) {
    st = launch_zero_fill(base, kScratchBytes, s);
    if (st != I4D_OK) {
      std::lock_guard<std::mutex> lock(g_mu);
      g_cleared[dev] = false;
      return st;
    }
  }
  return run_decode_step(layer, cache, x_in, x_out, ctx_len, M, max_ctx_len, num_splits, (char*)base, wl,
                         split_part_bytes, attn_f32, s, kFmtInt4);
}
