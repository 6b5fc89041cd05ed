// bf16-input chunkwise kernels, d_k in {128}, chunk in {32, 64, 128, 256, 512}, d_v tiles of 64 (256 threads).
// Chunks longer than 64 tokens run as 64-token sub-chunks: the instances differ only in the segment plan.
#include "chunk_bf16.h"

namespace ret {

bool chunk_kernels_bf16_128(int dk, int dv, int C, ChunkKernels* out) {
    if (dv % 64) return false;
#define RET_CASE(DKv, Cv) \
    if (dk == DKv && C == Cv) { *out = chunk_entry_bf16<DKv, Cv>(); return true; }
    RET_CASE(128, 32)
    RET_CASE(128, 64)
    if (dk == 128 && (C == 128 || C == 256 || C == 512)) { *out = chunk_entry_bf16<128, 128>(); return true; }
#undef RET_CASE
    return false;
}

}  // namespace ret
