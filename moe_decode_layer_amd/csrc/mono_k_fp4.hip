/* libmonolayer: instantiations of the launches for routed experts in format FP4. */
#include "mono_kernels.h"

namespace mono {
template int launch_fmt<BF16, FP4, BF16, 1>(Kernel, const Params&, int, hipStream_t);
template int launch_fmt<BF16, FP4, BF16, kMaxRows>(Kernel, const Params&, int, hipStream_t);
template int launch_fmt<BF16, FP4, Q8, 1>(Kernel, const Params&, int, hipStream_t);
template int launch_fmt<BF16, FP4, Q8, kMaxRows>(Kernel, const Params&, int, hipStream_t);
template int launch_fmt<BF16, FP4, FP4, 1>(Kernel, const Params&, int, hipStream_t);
template int launch_fmt<BF16, FP4, FP4, kMaxRows>(Kernel, const Params&, int, hipStream_t);
}  // namespace mono
