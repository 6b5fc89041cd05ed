// Instances of the wide-head chunkwise kernels. This source is compiled with the MFMA accumulators held in
// architectural registers (build.py): the kernels' state is read back as MFMA operands every step, and
// accumulators in the accumulation registers would cost a move for each of those reads.
#include "chunk_dma_bf16.h"
#include "chunk_wide_bf16.h"

namespace ret {

static_assert(WideB<256>::NT == kWideThreads && WideB<128>::NT == kWideThreads, "workgroup size");
static_assert(WideB<256>::C == kWideStep && WideB<128>::C == kWideStep, "step");
static_assert(DmaB<256>::NT == kDmaThreads && DmaB<128>::NT == kDmaThreads, "workgroup size");
static_assert(DmaB<256>::DVT == kDmaDvt && DmaB<128>::DVT == kDmaDvt, "d_v tile");
static_assert(DmaB<256>::C == kDmaStep && DmaB<128>::C == kDmaStep, "step");

fwd_kernel_t chunk_wide_get(int dk, bool rev) {
    if (dk == 256) return rev ? chunk_wide_bf16<256, true> : chunk_wide_bf16<256, false>;
    if (dk == 128) return rev ? chunk_wide_bf16<128, true> : chunk_wide_bf16<128, false>;
    return nullptr;
}

bool chunk_dma_get(int dk, DmaKernels* out) {
    if (dk == 256) {
        *out = {chunk_dma_local_bf16<256, false>, unit_scan_kernel<256>, chunk_dma_full_bf16<256, false>,
                chunk_dma_local_bf16<256, true>, chunk_dma_full_bf16<256, true>};
        return true;
    }
    if (dk == 128) {
        *out = {chunk_dma_local_bf16<128, false>, unit_scan_kernel<128>, chunk_dma_full_bf16<128, false>,
                chunk_dma_local_bf16<128, true>, chunk_dma_full_bf16<128, true>};
        return true;
    }
    return false;
}

}  // namespace ret
