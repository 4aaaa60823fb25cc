// Persistent-kernel instantiations for the MoE decoder (VALU).
#include "megakernel_impl.h"

namespace mk {
const void* kernel_moe(int B, int hd) { return kernel_of<false, true>(B, hd); }
}  // namespace mk
