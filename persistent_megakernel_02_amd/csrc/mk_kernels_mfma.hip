// Persistent-kernel instantiations for the dense decoder with the matrix-core GEMV.
#include "megakernel_impl.h"

namespace mk {
const void* kernel_mfma(int B, int hd) { return kernel_of<true, false>(B, hd); }
}  // namespace mk
