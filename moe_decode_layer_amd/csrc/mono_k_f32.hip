/* libmonolayer: instantiations of the launches for routed experts in format F32. */
#include "mono_kernels.h"

namespace mono {
template int launch_fmt<F32, F32, F32, 1>(Kernel, const Params&, int, hipStream_t);
template int launch_fmt<F32, F32, F32, kMaxRows>(Kernel, const Params&, int, hipStream_t);
}  // namespace mono
