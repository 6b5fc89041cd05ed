// bf16-input chunkwise kernels, d_k in {32, 64}, chunk in {32, 64, 128, 256, 512}, d_v tiles of 64. Chunks
// longer than 64 tokens run as 64-token sub-chunks: the instances differ only in the segment plan.
#include "chunk_seg_bf16.h"

namespace ret {

// The single-pass kernels, plus the on-chip variant for short segments. The on-chip kernel runs 32-token
// sub-chunks whatever the chunk: its segment is on chip anyway, and shorter steps bring each chunk's first
// products and the segment's aggregate earlier (retention-layer-d512: 26.0 against 27.3 us per call; 38 against
// 42 us MALL-cold).
template <int DK, int C>
ChunkKernels chunk_entry_small() {
    constexpr int CS = 32;
    ChunkKernels k = chunk_entry_bf16<DK, C>();
    k.seg = chunk_seg_bf16<DK, CS, false>;
    // (the PRE instances serve the gradients: v rows rotated while staged, outputs turned back)
    k.seg_pre = chunk_seg_bf16<DK, CS, true, false, true>;
    k.seg_rev = chunk_seg_bf16<DK, CS, true, true, true>;
    k.seg_rot_rev = chunk_seg_bf16<DK, CS, false, true>;
    k.seg_tokens = SegB<DK, CS, false>::RT;
    return k;
}

bool chunk_kernels_bf16_small(int dk, int dv, int C, ChunkKernels* out) {
    if (dv % 64) return false;
#define RET_CASE(DKv, Cv) \
    if (dk == DKv && C == Cv) { *out = chunk_entry_small<DKv, Cv>(); return true; }
    RET_CASE(32, 32)
    RET_CASE(32, 64)
    RET_CASE(64, 32)
    RET_CASE(64, 64)
    if ((dk == 32 || dk == 64) && (C == 128 || C == 256 || C == 512)) {
        *out = dk == 32 ? chunk_entry_small<32, 128>() : chunk_entry_small<64, 128>();
        return true;
    }
#undef RET_CASE
    return false;
}

}  // namespace ret
