// Parallel-form, decode-step and segment-scan kernel instances.
#include "kernels.h"

namespace ret {

// ---------------------------------------------------------------------------------------------------
// segment_scan: per (b, h), W[0] = state_in (or 0); W[g] = gamma^seg_len W[g-1] + W[g] for g = 1..nseg-1,
// where W[g] held the local end state of segment g - 1. Elementwise over d_k x d_v, sequential over g. The
// loads of a group of segments are issued together before the dependent chain runs, so the chain costs one
// memory round trip per group rather than one per segment.
// ---------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void segment_scan_kernel(FwdArgs a) {
    constexpr int G = 16;  // segments loaded per round trip
    const int pair = blockIdx.y;
    const long long per = (long long)a.dk * a.dv;
    const long long e = ((long long)blockIdx.x * kThreads + threadIdx.x) * 4;
    if (e >= per) return;
    const float decay = __builtin_amdgcn_exp2f((float)a.seg_len * a.log2g[pair % a.H]);
    float* W = a.ws + (long long)pair * a.nseg * per + e;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.state_in) acc = *reinterpret_cast<const float4*>(a.state_in + (long long)pair * per + e);
    *reinterpret_cast<float4*>(W) = acc;
    for (int g0 = 1; g0 < a.nseg; g0 += G) {
        float4 u[G];
#pragma unroll
        for (int j = 0; j < G; ++j)  // branch-free: past the last segment re-read the last one (unused)
            u[j] = *reinterpret_cast<const float4*>(W + (long long)min(g0 + j, a.nseg - 1) * per);
#pragma unroll
        for (int j = 0; j < G; ++j)
            if (g0 + j < a.nseg) {
                acc.x = decay * acc.x + u[j].x;
                acc.y = decay * acc.y + u[j].y;
                acc.z = decay * acc.z + u[j].z;
                acc.w = decay * acc.w + u[j].w;
                *reinterpret_cast<float4*>(W + (long long)(g0 + j) * per) = acc;
            }
    }
}

// ---------------------------------------------------------------------------------------------------
// slot_scan: the states entering the segments of a split run. Slot 0 of each unit holds W_0 (state_in, or zero),
// slot s >= 1 the local end state of segment s - 1, each in one layout (the same in every slot); W_s =
// gamma^seg_len W_(s-1) + slot s replaces slot s. Elementwise: one thread per 2 consecutive floats of a slot of
// gridDim.x * 512 floats (many small workgroups: the chain over the segments is latency-bound); grid.y = the
// units, d_v tiles of each (b, h) consecutive. The loads of a group of 16 segments are issued together.
// ---------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void slot_scan_kernel(FwdArgs a) {
    constexpr int G = 16;
    const long long per = (long long)gridDim.x * 512;
    const int unit = blockIdx.y, ntiles = gridDim.y / (a.B * a.H);
    const float decay = __builtin_amdgcn_exp2f((float)a.seg_len * a.log2g[unit / ntiles % a.H]);
    float* W = a.ws + (long long)unit * a.nseg * per + ((long long)blockIdx.x * 256 + threadIdx.x) * 2;
    float2 acc = *reinterpret_cast<const float2*>(W);
    for (int g0 = 1; g0 < a.nseg; g0 += G) {
        float2 u[G];
#pragma unroll
        for (int j = 0; j < G; ++j)  // branch-free: past the last segment re-read the last one (unused)
            u[j] = *reinterpret_cast<const float2*>(W + (long long)min(g0 + j, a.nseg - 1) * per);
#pragma unroll
        for (int j = 0; j < G; ++j)
            if (g0 + j < a.nseg) {
                acc.x = decay * acc.x + u[j].x;
                acc.y = decay * acc.y + u[j].y;
                *reinterpret_cast<float2*>(W + (long long)(g0 + j) * per) = acc;
            }
    }
}

// ---------------------------------------------------------------------------------------------------
// rotate_qk: q' = rotated q, k' = rotated k (bf16 in, bf16 out), the rotation the chunk kernels otherwise
// apply while staging. Written once when a call stages the same rows for several d_v tiles. Thread: one
// 16-byte segment (8 dims, 4 pairs) of one (b, h) row over kRotTokens consecutive tokens; the factors of the
// first token are evaluated exactly, later ones by angle addition with the one-token step. All of a thread's
// q and k rows are requested before the first is used (2 kRotTokens 16-byte loads in flight per thread instead
// of two): the kernel streams, and what bounds it is the bytes in flight. The loads carry the non-temporal hint
// (each row is read once here; the chunk kernels read q' and k', not q and k).
// ---------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rotate_qk_kernel(FwdArgs a) {
    const int segs = a.H * a.dk / 8;  // segments of one token's row over all heads
    const int nblk = (a.N + kRotTokens - 1) / kRotTokens;
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (long long)a.B * nblk * segs) return;
    const int r = (int)(gid % segs);
    const long long bt = gid / segs;
    const int b = (int)(bt / nblk), n0 = (int)(bt % nblk) * kRotTokens;
    const int h = r / (a.dk / 8), pair0 = (r % (a.dk / 8)) * 4;
    const long long row = (long long)a.H * a.dk;  // elements between tokens
    const long long base = (((long long)b * a.N + n0) * a.H + h) * a.dk + pair0 * 2;
    const int nt = min(kRotTokens, a.N - n0);
    // rows past the sequence's end (a partial last block) re-read its last row and are not stored
    u32x4_t uq[kRotTokens], uk[kRotTokens];
#pragma unroll
    for (int i = 0; i < kRotTokens; ++i) {
        const long long off = base + (long long)min(i, nt - 1) * row;
        uq[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>((const uint16_t*)a.q + off));
        uk[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>((const uint16_t*)a.k + off));
    }
    float c[4], s[4], dc[4], ds[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        rot_cs(a.pos0 + n0, a.theta[pair0 + j], &c[j], &s[j]);
        rot_cs(1, a.theta[pair0 + j], &dc[j], &ds[j]);
    }
#pragma unroll
    for (int i = 0; i < kRotTokens; ++i) {
        float fq[8], fk[8];
        unpack8_bf16(make_uint4(uq[i][0], uq[i][1], uq[i][2], uq[i][3]), fq);
        unpack8_bf16(make_uint4(uk[i][0], uk[i][1], uk[i][2], uk[i][3]), fk);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float q0 = fq[2 * j], q1 = fq[2 * j + 1], k0 = fk[2 * j], k1 = fk[2 * j + 1];
            fq[2 * j] = q0 * c[j] - q1 * s[j];
            fq[2 * j + 1] = q0 * s[j] + q1 * c[j];
            fk[2 * j] = k0 * c[j] - k1 * s[j];
            fk[2 * j + 1] = k0 * s[j] + k1 * c[j];
            const float nc = c[j] * dc[j] - s[j] * ds[j];
            s[j] = s[j] * dc[j] + c[j] * ds[j];
            c[j] = nc;
        }
        if (i < nt) {
            *reinterpret_cast<uint4*>((uint16_t*)a.qr + base + i * row) = pack8_bf16(fq);
            *reinterpret_cast<uint4*>((uint16_t*)a.kr + base + i * row) = pack8_bf16(fk);
        }
    }
}

fwd_kernel_t rotate_qk_get() { return rotate_qk_kernel; }

bool parallel_kernel_get(bool bf16_in, int dk, int dv, ParKernel* out) {
    if (!bf16_in) {
        if (dv % 16) return false;
        if (dk == 16) { *out = {parallel_kernel<F32, 16, 32, 16>, 32, 16}; return true; }
        if (dk == 32) { *out = {parallel_kernel<F32, 32, 32, 16>, 32, 16}; return true; }
        if (dk == 64) { *out = {parallel_kernel<F32, 64, 32, 16>, 32, 16}; return true; }
        return false;
    }
    if (dv % 64) return false;
    if (dk == 32) { *out = {parallel_kernel<BF16, 32, 64, 64>, 64, 64}; return true; }
    if (dk == 64) { *out = {parallel_kernel<BF16, 64, 64, 64>, 64, 64}; return true; }
    if (dk == 128) { *out = {parallel_kernel<BF16, 128, 64, 64>, 64, 64}; return true; }
    if (dk == 256) { *out = {parallel_kernel<BF16, 256, 64, 64>, 64, 64}; return true; }
    return false;
}

// Tiles of a decode workgroup: 64, 32 or 16 state columns per wave (more, smaller waves per (b, h) for more
// memory parallelism) and 64, 32 or 16 rows per wave (several waves per column tile). Every lane keeps at
// least one pair of rows: rows per lane = wr * cw / 256 >= 2. Workgroups hold one (b, h) pair, or as many as
// fill 8 waves (step_group_pairs).
namespace {
template <class E, int DK, int CW, int WR, bool POS = false>
step_kernel_t step_pick(bool grouped, bool nt) {
    if constexpr (WR <= DK && WR * CW >= 512 && DK / WR <= 16) {
        constexpr int G = step_group_pairs(DK, WR);
        if (grouped && G > 1)
            return nt ? recurrent_step_kernel<E, DK, CW, WR, G, POS, true> : recurrent_step_kernel<E, DK, CW, WR, G, POS, false>;
        return nt ? recurrent_step_kernel<E, DK, CW, WR, 1, POS, true> : recurrent_step_kernel<E, DK, CW, WR, 1, POS, false>;
    }
    return nullptr;
}
// Per-sequence positions: the default tile of each d_k (64 columns; 32 rows per wave, d_k rows below 32).
template <class E>
step_kernel_t step_pick_positions(int dk, bool grouped, bool nt) {
    switch (dk) {
        case 16: return step_pick<E, 16, 64, 16, true>(grouped, nt);
        case 32: return step_pick<E, 32, 64, 32, true>(grouped, nt);
        case 64: return step_pick<E, 64, 64, 32, true>(grouped, nt);
        case 128: return step_pick<E, 128, 64, 32, true>(grouped, nt);
        case 256: return step_pick<E, 256, 64, 32, true>(grouped, nt);
        default: return nullptr;
    }
}
template <class E, int DK, int CW>
step_kernel_t step_pick_wr(int wr, bool grouped, bool nt) {
    if (wr == 16) return step_pick<E, DK, CW, 16>(grouped, nt);
    if (wr == 32) return step_pick<E, DK, CW, 32>(grouped, nt);
    return step_pick<E, DK, CW, 64>(grouped, nt);
}
template <class E, int DK>
step_kernel_t step_pick_cw(int cw, int wr, bool grouped, bool nt) {
    if (cw == 16) return step_pick_wr<E, DK, 16>(wr, grouped, nt);
    if (cw == 32) return step_pick_wr<E, DK, 32>(wr, grouped, nt);
    return step_pick_wr<E, DK, 64>(wr, grouped, nt);
}
template <class E>
step_kernel_t step_pick_dk(int dk, int cw, int wr, bool grouped, bool nt) {
    switch (dk) {
        case 16: return step_pick_cw<E, 16>(cw, wr, grouped, nt);
        case 32: return step_pick_cw<E, 32>(cw, wr, grouped, nt);
        case 64: return step_pick_cw<E, 64>(cw, wr, grouped, nt);
        case 128: return step_pick_cw<E, 128>(cw, wr, grouped, nt);
        case 256: return step_pick_cw<E, 256>(cw, wr, grouped, nt);
        default: return nullptr;
    }
}
}  // namespace

step_kernel_t step_kernel_get(bool bf16_in, int dk, int dv, int npairs, int cw, int wr, int pairs_mode,
                              bool positions, bool stream, int* cw_used, int* wr_used, int* ppw_used) {
    if (cw == 0 || positions) cw = 64;  // defaults: 64 columns x 32 rows per wave (two waves per 64-row tile)
    if (wr == 0 || positions) wr = 32;
    if (cw != 16 && cw != 32 && cw != 64) return nullptr;
    if (wr != 16 && wr != 32 && wr != 64) return nullptr;
    if (wr > dk) wr = dk < 16 ? 16 : dk;                // short d_k: one wave holds every row
    while (wr * cw < 512 && cw < 64) cw *= 2;           // at least two rows per lane
    while (wr * cw < 512 && wr < 64 && wr < dk) wr *= 2;
    *cw_used = cw;
    *wr_used = wr;
    // Grouped workgroups where they still give every CU one: mode 0 decides, 1 forces one pair, 2 grouping. A
    // streamed state goes one pair per workgroup by default: its requests reach memory sooner from many small
    // workgroups.
    const int g = step_group_pairs(dk, wr);
    const long long wgs = (long long)(npairs + g - 1) / g * ((dv + cw - 1) / cw);
    const bool grouped = g > 1 && (pairs_mode == 2 || (pairs_mode == 0 && !stream && wgs >= 256));
    *ppw_used = grouped ? g : 1;
    if (positions)
        return bf16_in ? step_pick_positions<BF16>(dk, grouped, stream) : step_pick_positions<F32>(dk, grouped, stream);
    return bf16_in ? step_pick_dk<BF16>(dk, cw, wr, grouped, stream) : step_pick_dk<F32>(dk, cw, wr, grouped, stream);
}

fwd_kernel_t segment_scan_get() { return segment_scan_kernel; }
fwd_kernel_t slot_scan_get() { return slot_scan_kernel; }

}  // namespace ret
