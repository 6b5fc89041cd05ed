// bf16-input chunkwise kernels, d_k in {32, 64}, chunk in {32, 64, 128}, d_v tiles of 64.
#include "chunk_seg_bf16.h"

namespace ret {

// The single-pass kernels, plus the on-chip variant for short segments.
template <int DK, int C>
ChunkKernels chunk_entry_small() {
    constexpr int CI = C > 64 ? 64 : C;
    ChunkKernels k = chunk_entry_bf16<DK, C>();
    k.seg = chunk_seg_bf16<DK, CI, false>;
    k.seg_pre = chunk_seg_bf16<DK, CI, true>;
    k.seg_tokens = SegB<DK, CI, false>::RT;
    return k;
}

bool chunk_kernels_bf16_small(int dk, int dv, int C, ChunkKernels* out) {
    if (dv % 64) return false;
#define RET_CASE(DKv, Cv) \
    if (dk == DKv && C == Cv) { *out = chunk_entry_small<DKv, Cv>(); return true; }
    RET_CASE(32, 32)
    RET_CASE(32, 64)
    RET_CASE(32, 128)
    RET_CASE(64, 32)
    RET_CASE(64, 64)
    RET_CASE(64, 128)
#undef RET_CASE
    return false;
}

}  // namespace ret
