// bf16-input chunkwise kernels, d_k in {256}, chunk in {32, 64, 128, 256, 512} (chunks longer than 64 tokens
// run as 64-token sub-chunks: the instances differ only in the segment plan). Where d_v is a multiple of 128 the d_v
// tile is 128 columns: 512 threads whose waves own 16 columns each (the default: two waves per SIMD), or 256
// threads whose waves own 32 columns each (twice the operand reuse per LDS read, one wave per SIMD).
// `variant` picks 0: 512 x 16 (default), 1: 256 x 32, 2: the 256-thread kernel with 16-column waves and d_v
// tiles of 64. Other d_v: 256 threads with d_v tiles of 64.
#include "chunk_bf16.h"

namespace ret {

bool chunk_kernels_bf16_256(int dk, int dv, int C, int variant, ChunkKernels* out) {
    if (dv % 64) return false;
    int mode = variant == 1 ? 2 : variant == 2 ? 0 : 1;  // 0: 256 threads x 16 columns, 1: 512 x 16, 2: 256 x 32
    if (dv % 128) mode = 0;
#define RET_CASE(DKv, Cv)                                                                             \
    if (dk == DKv && C == Cv) {                                                                       \
        *out = mode == 1   ? chunk_entry_bf16<DKv, Cv, 512>()                                         \
               : mode == 2 ? chunk_entry_bf16<DKv, Cv, 256, 2>()                                      \
                           : chunk_entry_bf16<DKv, Cv, 256>();                                        \
        return true;                                                                                  \
    }
    RET_CASE(256, 32)
    RET_CASE(256, 64)
    if (C == 256 || C == 512) C = 128;
    RET_CASE(256, 128)
#undef RET_CASE
    return false;
}

}  // namespace ret
