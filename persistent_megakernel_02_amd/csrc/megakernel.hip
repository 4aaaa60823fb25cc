// Host-side launch of the persistent decode megakernel (page
// "斯坦福团队新作让Llama1B实现毫秒级推理获Karpathy盛赞", section
// "Megakernel：从零设计的深度融合方案": one launch per decode step).  The kernel
// templates live in megakernel_impl.h; each kind is instantiated in its own
// translation unit (mk_kernels_valu.hip, mk_kernels_mfma.hip, mk_kernels_moe.hip)
// so that a kernel carries only its own code paths.
#include <hip/hip_runtime.h>

#include "mk_internal.h"

namespace mk {

const void* kernel_valu(int B, int hd);
const void* kernel_mfma(int B, int hd);
const void* kernel_moe(int B, int hd);

size_t megakernel_lds_bytes(const Params& P) { return (size_t)P.ring_chunks * kChunk + P.x_bytes; }

hipError_t launch_megakernel(const Params& P, const StepArgs& A, hipStream_t stream) {
    const int kind = P.E > 0 ? 2 : P.gemv_mfma ? 1 : 0;
    const void* fn = kind == 2 ? kernel_moe(P.B, P.hd) : kind == 1 ? kernel_mfma(P.B, P.hd) : kernel_valu(P.B, P.hd);
    if (!fn) return hipErrorInvalidValue;
    // dynamic LDS above the default is allowed per kernel once
    static size_t configured[3][2][4] = {};
    const int bi = P.B == 1 ? 0 : P.B == 2 ? 1 : P.B == 4 ? 2 : 3;
    size_t& cfgd = configured[kind][P.hd == 128 ? 1 : 0][bi];
    const size_t lds = megakernel_lds_bytes(P);
    if (cfgd < lds) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        cfgd = lds;
    }
    void* args[] = {(void*)&P, (void*)&A};
    // A plain launch: one workgroup fills a compute unit's LDS, and the host
    // admits at most one workgroup per compute unit, so every workgroup of the
    // grid is resident at once.  (A cooperative launch guarantees the same but
    // measured about 18 us more between consecutive steps.)
    return hipLaunchKernel(fn, dim3(P.n_cu), dim3(kThreads), args, lds, stream);
}

bool megakernel_supports(int B, int hd) { return (B == 1 || B == 2 || B == 4 || B == 8) && (hd == 64 || hd == 128); }

}  // namespace mk
