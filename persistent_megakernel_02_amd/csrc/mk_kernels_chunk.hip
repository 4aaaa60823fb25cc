// Persistent-kernel instantiations for multi-position steps: kChunkRows rows of
// one sequence (a prompt chunk, or a token and its draft tokens) in one launch,
// VALU dot products, dense or MoE decoder.
#include "megakernel_impl.h"

namespace mk {
const void* kernel_chunk(int hd, bool moe) { return moe ? kernel_of_chunk<true>(hd) : kernel_of_chunk<false>(hd); }
}  // namespace mk
