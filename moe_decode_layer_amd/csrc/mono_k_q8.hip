/* libmonolayer: instantiations of the launches for routed experts in format Q8. */
#include "mono_kernels.h"

namespace mono {
MONO_INSTANTIATE(BF16, Q8, BF16)
MONO_INSTANTIATE(BF16, Q8, Q8)
MONO_INSTANTIATE(BF16, Q8, FP4)
}  // namespace mono
