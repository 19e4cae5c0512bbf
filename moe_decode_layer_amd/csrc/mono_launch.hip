/*
 * libmonolayer kernel dispatch: format-independent kernels, workspace helper kernels and the
 * mapping from (kernel, activation type, weight formats, rows) to an instantiated launch.
 * The format-specific launches are instantiated in mono_k_*.hip.
 */
#include "mono_kernels.h"

namespace mono {

#define MONO_FMT_EXTERN(A, RF, SF)                                                         \
  extern template int launch_fmt<A, RF, SF, 1>(Kernel, const Params&, int, hipStream_t);   \
  extern template int launch_fmt<A, RF, SF, kMaxRows>(Kernel, const Params&, int, hipStream_t); \
  extern template int occ_fmt<A, RF, SF, 1>();                                              \
  extern template int occ_fmt<A, RF, SF, kMaxRows>();
MONO_FMT_EXTERN(F32, F32, F32)
MONO_FMT_EXTERN(BF16, BF16, BF16)
MONO_FMT_EXTERN(BF16, BF16, Q8)
MONO_FMT_EXTERN(BF16, BF16, FP4)
MONO_FMT_EXTERN(BF16, Q8, BF16)
MONO_FMT_EXTERN(BF16, Q8, Q8)
MONO_FMT_EXTERN(BF16, Q8, FP4)
MONO_FMT_EXTERN(BF16, FP4, BF16)
MONO_FMT_EXTERN(BF16, FP4, Q8)
MONO_FMT_EXTERN(BF16, FP4, FP4)
#undef MONO_FMT_EXTERN

template <int ACT, int RMAX>
static int launch_act(Kernel k, const Params& p, int rfmt, int sfmt, int grid, hipStream_t st) {
  switch (k) {
    case K_MIX_PARTIALS: MONO_LAUNCH((k_mix_partials<ACT, RMAX>), grid);
    case K_HC_PRE: MONO_LAUNCH((k_hc_pre<ACT, RMAX>), 1);
    case K_ROUTER_LOGITS: MONO_LAUNCH((k_router_logits<ACT, RMAX>), grid);
    case K_SELECT: MONO_LAUNCH(k_select<0>, 1);
    case K_EXPAND: MONO_LAUNCH((k_expand<ACT, RMAX>), grid);
    default: break;
  }
  if constexpr (ACT == F32) {
    if (rfmt == F32 && sfmt == F32) return launch_fmt<ACT, F32, F32, RMAX>(k, p, grid, st);
    return (int)hipErrorInvalidValue;
  } else {
#define MONO_FMT_CASE(RF, SF) \
  if (rfmt == RF && sfmt == SF) return launch_fmt<ACT, RF, SF, RMAX>(k, p, grid, st);
    MONO_FMT_CASE(BF16, BF16)
    MONO_FMT_CASE(BF16, Q8)
    MONO_FMT_CASE(BF16, FP4)
    MONO_FMT_CASE(Q8, BF16)
    MONO_FMT_CASE(Q8, Q8)
    MONO_FMT_CASE(Q8, FP4)
    MONO_FMT_CASE(FP4, BF16)
    MONO_FMT_CASE(FP4, Q8)
    MONO_FMT_CASE(FP4, FP4)
#undef MONO_FMT_CASE
    return (int)hipErrorInvalidValue;
  }
}

/* Control words to their initial values, and the tagged regions (carry partials, router logit
 * parts) to tag 0, which no fused launch writes, so that values left by launches before the
 * init are never taken as current. */
__global__ void k_ws_init(uint32_t* ctl, uint64_t* tagged, size_t tag_words) {
  const int t = threadIdx.x;
  if (blockIdx.x == 0)
    for (int w = t; w < CTL_WORDS; w += blockDim.x) ctl[w] = (w == CTL_FAULT_WG) ? 0xFFFFFFFFu : 0u;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + t; i < tag_words;
       i += (size_t)gridDim.x * blockDim.x)
    tagged[i] = 0u;
}

__global__ void k_ws_debug(uint32_t* ctl, uint32_t spin, uint32_t fwg, uint32_t fph) {
  if (threadIdx.x == 0) {
    ctl[CTL_SPIN] = spin;
    ctl[CTL_FAULT_WG] = fwg;
    ctl[CTL_FAULT_PHASE] = fph;
  }
}

__global__ void k_ws_trace(uint32_t* ctl, uint32_t on) {
  if (threadIdx.x == 0) ctl[CTL_TRACE] = on;
}


int launch(Kernel k, const Params& p, int act, int rfmt, int sfmt, int grid, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (k == K_WS_INIT) {
    hipLaunchKernelGGL(k_ws_init, dim3(64), dim3(256), 0, st, p.ctl,
                       reinterpret_cast<uint64_t*>(p.carry_part), p.tag_words);
    return (int)hipGetLastError();
  }
  const bool one = p.R <= 1;
  if (act == F32)
    return one ? launch_act<F32, 1>(k, p, rfmt, sfmt, grid, st)
               : launch_act<F32, kMaxRows>(k, p, rfmt, sfmt, grid, st);
  return one ? launch_act<BF16, 1>(k, p, rfmt, sfmt, grid, st)
             : launch_act<BF16, kMaxRows>(k, p, rfmt, sfmt, grid, st);
}

int launch_debug(uint32_t* ctl, uint32_t spin, uint32_t fwg, uint32_t fph, void* stream) {
  hipLaunchKernelGGL(k_ws_debug, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), ctl,
                     spin, fwg, fph);
  return (int)hipGetLastError();
}

int launch_trace(uint32_t* ctl, uint32_t on, void* stream) {
  hipLaunchKernelGGL(k_ws_trace, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), ctl, on);
  return (int)hipGetLastError();
}

int max_active_persistent(int act, int rfmt, int sfmt, int rows) {
  const bool one = rows <= 1;
  if (act == F32) {
    if (rfmt == F32 && sfmt == F32) return one ? occ_fmt<F32, F32, F32, 1>() : occ_fmt<F32, F32, F32, kMaxRows>();
    return -1;
  }
  if (act != BF16) return -1;
#define MONO_OCC_CASE(RF, SF)          \
  if (rfmt == RF && sfmt == SF)         \
    return one ? occ_fmt<BF16, RF, SF, 1>() : occ_fmt<BF16, RF, SF, kMaxRows>();
  MONO_OCC_CASE(BF16, BF16)
  MONO_OCC_CASE(BF16, Q8)
  MONO_OCC_CASE(BF16, FP4)
  MONO_OCC_CASE(Q8, BF16)
  MONO_OCC_CASE(Q8, Q8)
  MONO_OCC_CASE(Q8, FP4)
  MONO_OCC_CASE(FP4, BF16)
  MONO_OCC_CASE(FP4, Q8)
  MONO_OCC_CASE(FP4, FP4)
#undef MONO_OCC_CASE
  return -1;
}

int grid_size_for_device(int device) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
    return 0;
  return cus < kMaxGrid ? cus : kMaxGrid;
}

}  // namespace mono
