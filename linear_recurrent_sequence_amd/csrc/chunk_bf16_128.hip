// bf16-input chunkwise kernels, d_k in {128}, chunk in {32, 64, 128, 256, 512}, d_v tiles of 64 (256 threads).
// Chunks longer than 64 tokens run as 64-token sub-chunks: the instances differ only in the segment plan.
#include "chunk_bf16.h"

namespace ret {

// The wide-head kernel on operands staged as given (d_v tiles of 128), with the 512-thread kernel of 128-column
// tiles rotating while staging where no workspace holds rotated copies.
template <int C>
ChunkKernels chunk_entry_wide128() {
    ChunkKernels k = chunk_entry_bf16<128, C, 512>();  // (d_v tiles of 128 for both kernels of the set)
    k.fused_pre = chunk_wide_get(128);
    k.fused_rev = chunk_wide_get(128, true);
    k.rev_step = kWideStep;
    k.threads_pre = kWideThreads;
    k.pre_always = 1;
    k.target_wgs = 512;
    k.pre_name = "ret_chunk_wide";
    return k;
}

bool chunk_kernels_bf16_128(int dk, int dv, int C, int variant, ChunkKernels* out) {
    if (dv % 64) return false;
    if (variant == 3 && dv % 128 == 0 && dk == 128 && (C == 32 || C == 64 || C == 128 || C == 256 || C == 512)) {
        *out = C == 32 ? chunk_entry_wide128<32>() : C == 64 ? chunk_entry_wide128<64>() : chunk_entry_wide128<128>();
        return true;
    }
#define RET_CASE(DKv, Cv) \
    if (dk == DKv && C == Cv) { *out = chunk_entry_bf16<DKv, Cv>(); return true; }
    RET_CASE(128, 32)
    RET_CASE(128, 64)
    if (dk == 128 && (C == 128 || C == 256 || C == 512)) { *out = chunk_entry_bf16<128, 128>(); return true; }
#undef RET_CASE
    return false;
}

}  // namespace ret
