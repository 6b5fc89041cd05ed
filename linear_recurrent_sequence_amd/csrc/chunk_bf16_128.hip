// bf16-input chunkwise kernels, d_k in {128}, chunk in {32, 64, 128, 256, 512}: d_v tiles of 128 (512 threads)
// where d_v is a multiple of 128, else of 64 (256 threads), and the wide-head kernel (variant 3).
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
    k.fused_orot = 0;
    k.rev_step = kWideStep;
    k.threads_pre = kWideThreads;
    k.pre_always = 1;
    k.target_wgs = 512;
    k.pre_name = "ret_chunk_wide";
    return k;
}

// The set in three launches for chained segments (local passes, scan, full passes): no workgroup waits on a chain.
ChunkKernels split_launches(ChunkKernels k) {
    k.fused_split = 1;
    return k;
}

bool chunk_kernels_bf16_128(int dk, int dv, int C, int variant, ChunkKernels* out) {
    if (dv % 64 || dk != 128) return false;
    const bool chunk_ok = C == 32 || C == 64 || C == 128 || C == 256 || C == 512;
    if (variant == 3 && dv % 128 == 0 && chunk_ok) {
        *out = C == 32 ? chunk_entry_wide128<32>() : C == 64 ? chunk_entry_wide128<64>() : chunk_entry_wide128<128>();
        return true;
    }
    // d_v tiles of 128 where d_v allows (the default, and 4: 512 threads x 16 columns; 1: 256 threads x 32
    // columns), else (and 2) tiles of 64 (256 threads x 16 columns). One tile per head stages each q and k row
    // once instead of twice: on long-sequence 221 us against 242 us per call.
    const int mode = dv % 128 ? 2 : variant == 1 ? 1 : variant == 2 ? 2 : 4;
    if (!chunk_ok) return false;
    const int c = C > 128 ? 128 : C;
#define RET_CASE(Cv)                                                                                          \
    if (c == Cv) {                                                                                            \
        *out = mode == 4   ? split_launches(chunk_entry_bf16<128, Cv, 512, 1, true>())                        \
               : mode == 1 ? chunk_entry_bf16<128, Cv, 256, 2>()                                              \
                           : chunk_entry_bf16<128, Cv>();                                                     \
        return true;                                                                                          \
    }
    RET_CASE(32)
    RET_CASE(64)
    RET_CASE(128)
#undef RET_CASE
    return false;
}

}  // namespace ret
