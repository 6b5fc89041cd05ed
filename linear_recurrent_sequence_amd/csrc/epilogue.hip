// Multi-scale retention epilogue ("Hybrid Architectures: RetNet and the Three Computation Paradigms", sections
// 8.4 and 9.1; the paper summary, "Gating mechanism"): y = swish(gate) (.) GroupNorm_h(o), with one GroupNorm
// group per head. Each (token, head) row of d_v values is standardized by its own mean and biased variance,
// then scaled and shifted per channel; swish(x) = x sigmoid(x).
//
// A group is spread over LPG consecutive lanes holding EPL = 8 consecutive values each (16 bytes of bf16), so a
// wave covers 64 / LPG groups per round and its loads of one group are one contiguous run. Each wave takes
// ROUNDS rounds of groups and issues the loads of all of them before any arithmetic, so enough bytes are in
// flight per CU. Mean and variance are reduced by shuffles within the group's lanes: two passes over the values
// in registers. The sigmoid runs on the hardware 2^x and reciprocal (swish_hw) and the inverse standard
// deviation on the hardware reciprocal square root: a precise exp and divide would make the kernel bound by
// vector ALU work rather than by memory.
#include "kernels.h"

namespace ret {

namespace {

template <int DV>
struct EpiTile {
    static constexpr int EPL = 8;           // values per lane
    static constexpr int LPG = DV / EPL;    // lanes per group
    static constexpr int GPW = 64 / LPG;    // groups per wave and round
    static constexpr int ROUNDS = 4;
    static constexpr int GPB = 4 * GPW * ROUNDS;  // groups per 256-thread workgroup
    static_assert(LPG >= 1 && LPG <= 64 && 64 % LPG == 0, "epilogue tile");
};

// 8 consecutive values at element offset i of an fp32 or bf16 array (16-byte vectors). The epilogue reads and
// writes every value once: its accesses carry the non-temporal hint.
__device__ __forceinline__ void load8(const void* p, long long i, bool bf16, float* f) {
    if (bf16) {
        const u32x4_t u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>((const uint16_t*)p + i));
        const uint32_t w[4] = {u[0], u[1], u[2], u[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[2 * e] = __uint_as_float(w[e] << 16);
            f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; e += 4) {
            const f32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>((const float*)p + i + e));
            f[e] = x[0];
            f[e + 1] = x[1];
            f[e + 2] = x[2];
            f[e + 3] = x[3];
        }
    }
}

template <int DV>
__global__ __launch_bounds__(256) void msr_epilogue_kernel(EpiArgs a) {
    typedef EpiTile<DV> T;
    constexpr int LPG = T::LPG, NR = T::ROUNDS;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c0 = (lane % LPG) * 8;  // first channel of this lane within the head
    long long gi[NR], i0[NR];
    float x[NR][8], gv[NR][8];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        gi[r] = (long long)blockIdx.x * T::GPB + (r * 4 + w) * T::GPW + lane / LPG;
        const long long g = gi[r] < a.groups ? gi[r] : a.groups - 1;  // idle lanes read the last group
        i0[r] = g * DV + c0;
        load8(a.o, i0[r], a.o_bf16, x[r]);
        if (a.gate) load8(a.gate, i0[r], a.gate_bf16, gv[r]);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        group_standardize<LPG, 8>(x[r], (float)DV, a.eps);
        const int g = (int)(gi[r] < a.groups ? gi[r] : a.groups - 1);  // groups < 2^31 (checked on the host)
        const int ch = g % a.H * DV + c0;                                // channel of the concatenated heads
        if (a.weight) {
#pragma unroll
            for (int e = 0; e < 8; e += 4) {
                const float4 wv = *reinterpret_cast<const float4*>(a.weight + ch + e);
                x[r][e] *= wv.x;
                x[r][e + 1] *= wv.y;
                x[r][e + 2] *= wv.z;
                x[r][e + 3] *= wv.w;
            }
        }
        if (a.bias) {
#pragma unroll
            for (int e = 0; e < 8; e += 4) {
                const float4 bv = *reinterpret_cast<const float4*>(a.bias + ch + e);
                x[r][e] += bv.x;
                x[r][e + 1] += bv.y;
                x[r][e + 2] += bv.z;
                x[r][e + 3] += bv.w;
            }
        }
        if (a.gate) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[r][e] *= swish_hw(gv[r][e]);
        }
        if (gi[r] >= a.groups) continue;
        if (a.y_bf16) {
            __builtin_nontemporal_store(u32x4_t{pack2_bf16(x[r][0], x[r][1]), pack2_bf16(x[r][2], x[r][3]),
                                                pack2_bf16(x[r][4], x[r][5]), pack2_bf16(x[r][6], x[r][7])},
                                        reinterpret_cast<u32x4_t*>((uint16_t*)a.y + i0[r]));
        } else {
#pragma unroll
            for (int e = 0; e < 8; e += 4)
                __builtin_nontemporal_store(f32x4_t{x[r][e], x[r][e + 1], x[r][e + 2], x[r][e + 3]},
                                            reinterpret_cast<f32x4_t*>((float*)a.y + i0[r] + e));
        }
    }
}

template <int DV>
epi_kernel_t epi_pick(int* gpw) {
    *gpw = EpiTile<DV>::GPB;
    return msr_epilogue_kernel<DV>;
}

}  // namespace

epi_kernel_t epilogue_kernel_get(int dv, int* groups_per_wg) {
    switch (dv) {
        case 16: return epi_pick<16>(groups_per_wg);
        case 32: return epi_pick<32>(groups_per_wg);
        case 64: return epi_pick<64>(groups_per_wg);
        case 128: return epi_pick<128>(groups_per_wg);
        case 256: return epi_pick<256>(groups_per_wg);
        case 512: return epi_pick<512>(groups_per_wg);
        default: return nullptr;
    }
}

}  // namespace ret
