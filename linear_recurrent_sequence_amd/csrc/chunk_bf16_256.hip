// bf16-input chunkwise kernels, d_k in {256}, chunk in {32, 64, 128}: workgroups of 512 threads with d_v tiles
// of 128 where d_v allows it (RET_DK256_THREADS=256 asks for the 256-thread kernels), else 256 threads with
// d_v tiles of 64.
#include <stdlib.h>

#include "chunk_bf16.h"

namespace ret {

bool chunk_kernels_bf16_256(int dk, int dv, int C, ChunkKernels* out) {
    if (dv % 64) return false;
    const char* env = getenv("RET_DK256_THREADS");
    const bool wide = dv % 128 == 0 && !(env && atoi(env) == 256);
#define RET_CASE(DKv, Cv)                                                                   \
    if (dk == DKv && C == Cv) {                                                             \
        *out = wide ? chunk_entry_bf16<DKv, Cv, 512>() : chunk_entry_bf16<DKv, Cv, 256>(); \
        return true;                                                                        \
    }
    RET_CASE(256, 32)
    RET_CASE(256, 64)
    RET_CASE(256, 128)
#undef RET_CASE
    return false;
}

}  // namespace ret
