// Host-side launch of the persistent decode megakernel (page
// "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞", section
// "Megakernel：从零设计的深度融合方案": one launch per decode step).  The kernel
// templates live in megakernel_impl.h; each kind is instantiated in its own
// translation unit (mk_kernels_valu.hip, mk_kernels_mfma.hip, mk_kernels_moe.hip,
// mk_kernels_chunk.hip) so that a kernel carries only its own code paths.
#include <hip/hip_runtime.h>

#include "mk_internal.h"

namespace mk {

const void* kernel_valu(int B, int hd);
const void* kernel_mfma(int B, int hd);
const void* kernel_moe(int B, int hd);
const void* kernel_chunk(int hd, bool moe);

size_t megakernel_lds_bytes(const Params& P) { return (size_t)P.ring_chunks * kChunk + P.x_bytes; }

static const void* megakernel_fn(const Params& P) {
    if (P.chunk) return P.B == kChunkRows && !P.gemv_mfma ? kernel_chunk(P.hd, P.E > 0) : nullptr;
    const int kind = P.E > 0 ? 2 : P.gemv_mfma ? 1 : 0;
    return kind == 2 ? kernel_moe(P.B, P.hd) : kind == 1 ? kernel_mfma(P.B, P.hd) : kernel_valu(P.B, P.hd);
}

// Once per handle, on the current device: allow the kernel its dynamic LDS and
// check that one workgroup of it fits a compute unit.  The persistent kernel
// needs every one of its n_cu workgroups resident at once (they wait on each
// other's values); with at most one workgroup per compute unit and no more
// workgroups than compute units that holds on an otherwise idle device.  Work
// that another stream runs on the same device at the same time can keep a
// compute unit busy; the device watchdog then ends the step with
// MK_E_DEVICE_TIMEOUT instead of letting it hang.
hipError_t prepare_megakernel(const Params& P) {
    const void* fn = megakernel_fn(P);
    if (!fn) return hipErrorInvalidValue;
    const size_t lds = megakernel_lds_bytes(P);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds);
    if (e != hipSuccess) return e;
    return per_cu >= 1 ? hipSuccess : hipErrorInvalidConfiguration;
}

hipError_t launch_megakernel(const Params& P, const StepArgs& A, hipStream_t stream) {
    const void* fn = megakernel_fn(P);
    if (!fn) return hipErrorInvalidValue;
    void* args[] = {(void*)&P, (void*)&A};
    // A plain launch: one workgroup fills a compute unit's LDS, and the host
    // admits at most one workgroup per compute unit, so every workgroup of the
    // grid is resident at once.  (A cooperative launch guarantees the same but
    // measured about 18 us more between consecutive steps.)
    return hipLaunchKernel(fn, dim3(P.n_cu), dim3(kThreads), args, megakernel_lds_bytes(P), stream);
}

bool megakernel_supports(int B, int hd) { return (B == 1 || B == 2 || B == 4 || B == 8) && (hd == 64 || hd == 128); }

}  // namespace mk
