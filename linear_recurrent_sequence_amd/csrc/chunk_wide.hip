// Instances of the wide-head chunkwise kernel. This source is compiled with the MFMA accumulators held in
// architectural registers (build.py): the kernel's state is read back as MFMA operands every step, and
// accumulators in the accumulation registers would cost a move for each of those reads.
#include "chunk_wide_bf16.h"

namespace ret {

static_assert(WideB<256>::NT == kWideThreads && WideB<128>::NT == kWideThreads, "workgroup size");

fwd_kernel_t chunk_wide_get(int dk) {
    if (dk == 256) return chunk_wide_bf16<256>;
    if (dk == 128) return chunk_wide_bf16<128>;
    return nullptr;
}

}  // namespace ret
