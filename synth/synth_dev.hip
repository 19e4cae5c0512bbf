/*
 * Seeded synthetic inputs, device build. Test and benchmark infrastructure:
 * fills device buffers with the streams defined in synth_core.h, byte for byte
 * the same as the host build (the equality is a GPU test). Used to create the
 * multi-gigabyte expert tensors in place instead of uploading them.
 *
 * Build: hipcc --offload-arch=gfx950 -O3 -ffp-contract=off -fPIC -shared
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth_core.h"

__global__ void __launch_bounds__(256) synth_fill_kernel(void* out, int kind, uint64_t key,
                                                         uint64_t first, uint64_t count, float p0,
                                                         float p1, int32_t i0, int32_t i1) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    syn_put(out, i, kind, key, first + i, p0, p1, i0, i1);
}

/* Enqueues the fill of out[0, count) on `stream`; returns a hipError_t code. */
extern "C" int synth_fill_device(void* out, int kind, uint64_t key, uint64_t first,
                                 uint64_t count, float p0, float p1, int32_t i0, int32_t i1,
                                 void* stream) {
  if (kind < SYN_F32_NORMAL || kind > SYN_E8M0) return (int)hipErrorInvalidValue;
  if (count == 0) return 0;
  uint64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(synth_fill_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, out, kind, key, first, count, p0, p1, i0, i1);
  return (int)hipGetLastError();
}
