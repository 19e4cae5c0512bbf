/* libmonolayer: instantiations of the launches for routed experts in format BF16. */
#include "mono_kernels.h"

namespace mono {
MONO_INSTANTIATE(BF16, BF16, BF16)
MONO_INSTANTIATE(BF16, BF16, Q8)
MONO_INSTANTIATE(BF16, BF16, FP4)
}  // namespace mono
