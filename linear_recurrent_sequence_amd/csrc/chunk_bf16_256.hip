// bf16-input chunkwise kernels, d_k in {256}, chunk in {32, 64, 128, 256, 512} (chunks longer than 64 tokens
// run as 64-token sub-chunks: the instances differ only in the segment plan). `variant` picks
//   0 (default): variant 5 where d_v is a multiple of 256, else variant 3 where d_v is a multiple of 128, else
//      the 256-thread kernel with d_v tiles of 64;
//   3: the wide-head kernel (four waves of 32 columns, 32-token steps, operands staged through registers, q and
//      k rotated once up front);
//   5: the LDS-loading wide-head kernels (d_v a multiple of 256: local passes, a scan of their states and the
//      full pass, eight waves of 32 columns, operands loaded straight into the LDS; with rotation and no room for
//      rotated copies in the workspace, variant 4);
//   1: the chained kernel with 256 threads x 32 columns; 2: the 256-thread kernel with 16-column waves and d_v
//   tiles of 64; 4 (or any other): the chained kernel with 512 threads x 16 columns (two waves per SIMD).
#include "chunk_bf16.h"

namespace ret {

// The wide-head kernel (256 threads, waves of 32 columns, 32-token steps) on operands staged as given, with the
// 512-thread kernel rotating while staging where no workspace holds rotated copies.
template <int C>
ChunkKernels chunk_entry_wide256() {
    ChunkKernels k = chunk_entry_bf16<256, C, 512>();
    k.fused_pre = chunk_wide_get(256);
    k.fused_rev = chunk_wide_get(256, true);
    k.fused_orot = 0;
    k.rev_step = kWideStep;
    k.threads_pre = kWideThreads;
    k.pre_always = 1;
    k.pre_name = "ret_chunk_wide";
    return k;
}

// The LDS-loading wide-head kernels alone (they only stage operands as given): local pass, scan, full pass.
template <int C>
ChunkKernels chunk_entry_dma256() {
    ChunkKernels k = chunk_entry_bf16<256, C, 512>();
    DmaKernels d;
    chunk_dma_get(256, &d);
    k.fused = k.fused_pre = d.full;
    k.fused_orot = 0;
    k.split_local = d.local;
    k.split_scan = d.scan;
    k.split_local_rev = d.local_rev;
    k.split_full_rev = d.full_rev;
    k.dvt = kDmaDvt;
    k.threads = k.threads_pre = kDmaThreads;
    k.pre_always = 1;
    k.pre_only = 1;
    k.fallback_variant = 4;
    k.target_wgs = 256;  // one workgroup per CU
    k.pre_name = "ret_chunk_dma";
    return k;
}

bool chunk_kernels_bf16_256(int dk, int dv, int C, int variant, ChunkKernels* out) {
    if (dv % 64) return false;
    const bool chunk_ok = C == 32 || C == 64 || C == 128 || C == 256 || C == 512;
    if ((variant == 0 || variant == 5) && dv % kDmaDvt == 0 && dk == 256 && chunk_ok) {
        *out = C == 32 ? chunk_entry_dma256<32>() : C == 64 ? chunk_entry_dma256<64>() : chunk_entry_dma256<128>();
        return true;
    }
    if ((variant == 0 || variant == 3) && dv % 128 == 0 && dk == 256 && chunk_ok) {
        *out = C == 32 ? chunk_entry_wide256<32>() : C == 64 ? chunk_entry_wide256<64>() : chunk_entry_wide256<128>();
        return true;
    }
    // 0: 256 threads x 16 columns, 1: 512 x 16 (variant 4), 2: 256 x 32
    int mode = variant == 1 ? 2 : variant == 2 ? 0 : 1;
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
