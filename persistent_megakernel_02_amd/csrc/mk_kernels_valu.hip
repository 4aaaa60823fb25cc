// Persistent-kernel instantiations for the dense decoder with VALU dot products.
#include "megakernel_impl.h"

namespace mk {
const void* kernel_valu(int B, int hd) { return kernel_of<false, false>(B, hd); }
}  // namespace mk
