// fp32-input chunkwise kernels (d_k in {16, 32, 64}, chunk in {16, 32, 64}, d_v tiles of 16).
#include "kernels.h"

namespace ret {

bool chunk_kernels_f32(int dk, int dv, int C, ChunkKernels* out) {
    if (dv % 16) return false;
#define RET_CASE(DKv, Cv) \
    if (dk == DKv && C == Cv) { *out = chunk_entry<F32, DKv, Cv, 16>(); return true; }
    RET_CASE(16, 16) RET_CASE(16, 32) RET_CASE(16, 64)
    RET_CASE(32, 16) RET_CASE(32, 32) RET_CASE(32, 64)
    RET_CASE(64, 16) RET_CASE(64, 32) RET_CASE(64, 64)
#undef RET_CASE
    return false;
}

}  // namespace ret
