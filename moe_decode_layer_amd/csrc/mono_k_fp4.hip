/* libmonolayer: instantiations of the launches for routed experts in format FP4. */
#include "mono_kernels.h"

namespace mono {
MONO_INSTANTIATE(BF16, FP4, BF16)
MONO_INSTANTIATE(BF16, FP4, Q8)
MONO_INSTANTIATE(BF16, FP4, FP4)
}  // namespace mono
