/* libmonolayer: instantiations of the launches for routed experts in format F32. */
#include "mono_kernels.h"

namespace mono {
MONO_INSTANTIATE(F32, F32, F32)
}  // namespace mono
