// paged_attn_decode for callers that cannot allocate device memory: the
// split-K partial states go to a static device array of this library instead
// of a caller-provided workspace.  The kernels are the decode's own; only the
// workspace pointer differs.
//
// The array is a device symbol.  In host code its name is only a host-side
// stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept; every later use
// (the kernels' workspace argument) takes that address.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "pa_internal.h"

namespace {

static_assert(PA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");

// Split-K scratch: float32 o, m and l of every (output row, split), laid out
// as the decode's workspace.  One copy per GPU, resident until the process
// ends.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, set once

pa_status noalloc_fail(pa_status st, const char* what) {
  pa::set_last_error(what);
  return st;
}

// Device address of this device's copy of `scratch`, looked up on first use.
pa_status scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      char buf[256];
      snprintf(buf, sizeof buf, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev, hipGetErrorString(e));
      return noalloc_fail(PA_ERR_LAUNCH, buf);
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status paged_attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, const int32_t* seq_lens, int32_t B, float scale,
                                    float* out, hipStream_t stream, const pa_dims* dims) {
  pa::set_last_error("");
  if (!dims) return noalloc_fail(PA_ERR_INVALID_ARG, "dims is NULL");
  int32_t P = 0;
  size_t need = 0;
  const pa_status st = paged_attn_plan(dims, B, &P, &need);
  if (st != PA_OK) return st;
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES) {
    char buf[256];
    snprintf(buf, sizeof buf,
             "%d splits need %zu bytes of partial states; the static scratch holds %d (use paged_attn_decode with a "
             "workspace, or fewer splits)",
             P, need, PA_NOALLOC_SCRATCH_BYTES);
    return noalloc_fail(PA_ERR_WORKSPACE, buf);
  }
  pa_dims d = *dims;
  d.workspace = nullptr;
  d.workspace_bytes = 0;
  if (dims->num_seqs > 0) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur < 0 || cur >= kMaxDevices)
      return noalloc_fail(PA_ERR_LAUNCH, "no current HIP device (or its index is 64 or more)");
    if (stream) {
      int sdev = -1;
      if (hipStreamGetDevice(stream, &sdev) != hipSuccess)
        return noalloc_fail(PA_ERR_INVALID_ARG, "hipStreamGetDevice failed on the stream");
      if (sdev != cur) {
        char buf[128];
        snprintf(buf, sizeof buf, "the stream belongs to device %d, the current device is %d", sdev, cur);
        return noalloc_fail(PA_ERR_INVALID_ARG, buf);
      }
    }
    void* ptr = nullptr;
    const pa_status sst = scratch_address(cur, &ptr);
    if (sst != PA_OK) return sst;
    d.workspace = ptr;
    d.workspace_bytes = PA_NOALLOC_SCRATCH_BYTES;
  }
  return paged_attn_decode(q, k_pool, v_pool, block_tables, seq_lens, B, scale, out, stream, &d);
}

}  // extern "C"
