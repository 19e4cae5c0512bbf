/*
 * libmonolayer: the fused layer-half launch for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). Its workspace is a
 * file-scope device array of fixed size, one copy per GPU for the life of the process.
 *
 * Host code never passes the array's name to a kernel or a copy: the name is a host-side
 * stand-in. Its device address is read once per device with hipGetSymbolAddress (that device
 * current) and kept; that address is what the launch receives.
 */
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "mono_internal.h"

static constexpr size_t kStaticBytes = (size_t)MONO_STATIC_WS_BYTES;

/* the workspace of every call of mono_ffn_layer_static on a device (one copy per device) */
static __device__ __align__(256) unsigned char scratch[kStaticBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_ptr[kMaxDevices];          /* device address of scratch on each device */
bool g_init[kMaxDevices];          /* an init was enqueued for g_shape[dev] */
mono_shape g_shape[kMaxDevices];   /* shape of the last launch on each device */

}  // namespace

extern "C" mono_status mono_ffn_layer_static(const mono_shape* shape, const mono_layer* layer,
                                             const float* w_mix_next, const void* state_in,
                                             const float* carry_in, void* state_out,
                                             float* carry_out, void* stream) {
  /* size first (host only): shapes whose workspace exceeds the array are refused */
  const size_t need = mono_workspace_bytes(shape);
  if (need == 0) return MONO_E_INVAL; /* mono_last_error lists the failed shape checks */
  if (need > kStaticBytes) {
    mono::set_last_error("the shape needs a workspace of %zu bytes, more than the %zu bytes of "
                         "the static workspace", need, kStaticBytes);
    return MONO_E_UNSUPPORTED;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    mono::set_last_error("no HIP device (or device index >= %d)", kMaxDevices);
    return MONO_E_DEVICE;
  }
  void* ws = nullptr;
  bool need_init = false;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        mono::set_last_error("hipGetSymbolAddress of the static workspace on device %d: %s", dev,
                             hipGetErrorString(e));
        return MONO_E_DEVICE;
      }
      g_ptr[dev] = p;
    }
    ws = g_ptr[dev];
    if (shape->rows > 0 &&
        (!g_init[dev] || std::memcmp(&g_shape[dev], shape, sizeof(mono_shape)) != 0)) {
      need_init = true;
      g_shape[dev] = *shape;
      g_init[dev] = true;
    }
  }
  if (need_init) {
    /* a kernel clears the counters and tagged regions for this shape (no memset node) */
    const mono_status st = mono_workspace_init(ws, shape, stream);
    if (st != MONO_OK) {
      std::lock_guard<std::mutex> lock(g_mu);
      g_init[dev] = false;
      return st;
    }
  }
  return mono_ffn_layer(shape, layer, w_mix_next, state_in, carry_in, state_out, carry_out, ws,
                        stream);
}
