// Kernel templates of libretention.so (gfx950). Each kernel-group source instantiates a subset and exposes
// getters; the C-ABI source launches them.
#pragma once

#include "retention_device.h"

namespace ret {

// Arguments shared by the chunk and parallel kernels (passed by value in the kernel-argument segment).
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    const float* state_in;   // [B,H,dk,dv] or null
    float* state_out;        // [B,H,dk,dv] or null
    float* ws;               // [B*H][nseg][dk][dv] segment states (split runs)
    int B, N, H, dk, dv;
    int nseg;                // segments per sequence
    int seg_len;             // tokens per segment (multiple of the chunk), last segment may be shorter
    int out_bf16;
    int rotate;
    long long pos0;
    float log2g[kMaxHeads];
    double theta[kMaxPairs];
};

// Tile lists. S tiles of a CxC chunk are the lower triangle (cb <= rb), enumerated row by row; tile i of any
// list belongs to wave i % 4 and lives in that wave's accumulator slot i / 4.
template <int NB>
struct Tri {
    static constexpr int count = NB * (NB + 1) / 2;
};

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------------------------------
// chunk_full: one workgroup per (segment, d_v tile, b*H + h). The segment's chunks are processed in stages
// (chunk, d_k slice); the global loads of stage i+1 are issued before stage i is computed.
// ---------------------------------------------------------------------------------------------------
template <class E, int DK, int C, int DVT>
struct FullCfg {
    typedef typename E::st st;
    static constexpr int KS = DK < 64 ? DK : 64;     // d_k slice staged at a time
    static constexpr int NSL = DK / KS;
    static constexpr int LDQ = KS + E::PAD;          // sQ, sK rows
    static constexpr int LDC = C + E::PAD;           // sKc, sVc, sP rows (token index contiguous)
    static constexpr int LDR = DK + E::PAD;          // sRt rows (d_k contiguous)
    static constexpr int LDO = DVT + 8;              // output tile rows (elements of the output type)
    static constexpr int NB = C / 16;                // row/col blocks of a chunk
    static constexpr int NDV = DVT / 16;             // d_v blocks
    static constexpr int NKB = DK / 16;              // d_k blocks
    static constexpr int NS = Tri<NB>::count;        // S tiles (lower triangle)
    static constexpr int NS_W = (NS + kWaves - 1) / kWaves;
    static constexpr int NO = NB * NDV;              // O tiles
    static constexpr int NO_W = (NO + kWaves - 1) / kWaves;
    static constexpr int NR = NKB * NDV;             // R tiles
    static constexpr int NR_W = (NR + kWaves - 1) / kWaves;
    static constexpr int UQ = (C / 8) * (KS / 8);    // staging units of Q (and of K) per slice
    static constexpr int UV = (C / 8) * (DVT / 8);   // staging units of V (first slice only)
    static constexpr int NU = (2 * UQ + UV + kThreads - 1) / kThreads;
    static constexpr int SQ = C * LDQ, SKC = KS * LDC, SVC = DVT * LDC, SP = C * LDC, SRT = DVT * LDR;
    // Region A holds sQ, sK and sKc while a chunk's slices are computed, then the output tile (fp32 at most).
    static constexpr int A_STAGE = (2 * SQ + SKC) * (int)sizeof(st), A_OUT = C * LDO * 4;
    static constexpr int A_BYTES = ((A_STAGE > A_OUT ? A_STAGE : A_OUT) + 15) / 16 * 16;
    static constexpr int LDS_BYTES = A_BYTES + (SVC + SP + SRT) * (int)sizeof(st);
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(C % 16 == 0 && DVT % 16 == 0 && DK % KS == 0 && KS % E::KD == 0 && C % E::KD == 0, "tiling");
};

template <class E, int DK, int C, int DVT>
__global__ __launch_bounds__(kThreads, 2) void chunk_full_kernel(FwdArgs a) {
    typedef FullCfg<E, DK, C, DVT> F;
    typedef typename E::st st;
    __shared__ __attribute__((aligned(16))) st smem[F::LDS_BYTES / sizeof(st)];
    st* sQ = smem;
    st* sK = sQ + F::SQ;
    st* sKc = sK + F::SQ;
    st* sVc = smem + F::A_BYTES / sizeof(st);
    st* sP = sVc + F::SVC;
    st* sRt = sP + F::SP;
    char* sO = reinterpret_cast<char*>(smem);  // output tile, over region A once a chunk's slices are done

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int seg = blockIdx.x, dvt = blockIdx.y, pair = blockIdx.z;
    const Seq s{a.N, a.H, pair / a.H, pair % a.H};
    const int dv0 = dvt * DVT;
    const float lg = a.log2g[s.h];
    const st* q = (const st*)a.q;
    const st* k = (const st*)a.k;
    const st* v = (const st*)a.v;
    const int osz = a.out_bf16 ? 2 : 4;

    // Scores above the diagonal are never written: keep them zero for the P.V product.
    for (int i = tid; i < F::SP; i += kThreads) sP[i] = (st)0;

    // Initial state for this segment: the segment-scan result, state_in, or zeros.
    const float* init = nullptr;
    if (a.nseg > 1)
        init = a.ws + ((long long)pair * a.nseg + seg) * DK * a.dv;
    else if (a.state_in)
        init = a.state_in + (long long)pair * DK * a.dv;
    f32x4_t R[F::NR_W];
#pragma unroll
    for (int i = 0; i < F::NR_W; ++i) {
        const int t = w + kWaves * i;
        R[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (t < F::NR && init) {
            const int rb = t / F::NDV, cb = t % F::NDV;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                R[i][e] = init[(long long)(rb * 16 + 4 * (lane >> 4) + e) * a.dv + dv0 + cb * 16 + (lane & 15)];
        }
    }
    // Copy of R (operand precision), transposed to [d_v][d_k], for the cross product.
#pragma unroll
    for (int i = 0; i < F::NR_W; ++i) {
        const int t = w + kWaves * i;
        if (t < F::NR) {
            const int rb = t / F::NDV, cb = t % F::NDV;
            store4(sRt + (cb * 16 + (lane & 15)) * F::LDR + rb * 16 + 4 * (lane >> 4), R[i]);
        }
    }

    const long long seg_t0 = (long long)seg * a.seg_len;
    const long long seg_t1 = min((long long)a.N, seg_t0 + a.seg_len);
    const int nst = (int)((seg_t1 - seg_t0 + C - 1) / C) * F::NSL;
    const long long qk_row0 = ((long long)s.b * a.N) * a.H + s.h;  // token 0 of this (b, h), in rows of d
    const int rsk = a.H * a.dk, rsv = a.H * a.dv;

    Raw<E> buf[F::NU];
    auto issue = [&](int i) {
        const long long t0 = seg_t0 + (long long)(i / F::NSL) * C;
        const int sl = i % F::NSL;
        const int L = (int)min((long long)C, seg_t1 - t0);
        const int total = 2 * F::UQ + (sl == 0 ? F::UV : 0);
#pragma unroll
        for (int j = 0; j < F::NU; ++j) {
            const int u = tid + kThreads * j;
            if (u < total) {
                const st* base;
                int rs, tb;
                if (u < 2 * F::UQ) {
                    const int x = u < F::UQ ? u : u - F::UQ;
                    tb = x / (F::KS / 8);
                    base = (u < F::UQ ? q : k) + (qk_row0 + t0 * a.H) * a.dk + sl * F::KS + (x % (F::KS / 8)) * 8;
                    rs = rsk;
                } else {
                    const int x = u - 2 * F::UQ;
                    tb = x / (DVT / 8);
                    base = v + (qk_row0 + t0 * a.H) * a.dv + dv0 + (x % (DVT / 8)) * 8;
                    rs = rsv;
                }
                issue_unit(buf[j], base + (long long)tb * 8 * rs, rs, L - tb * 8);
            }
        }
    };
    auto commit = [&](int i) {
        const long long t0 = seg_t0 + (long long)(i / F::NSL) * C;
        const int sl = i % F::NSL;
        const int L = (int)min((long long)C, seg_t1 - t0);
        const int total = 2 * F::UQ + (sl == 0 ? F::UV : 0);
#pragma unroll
        for (int j = 0; j < F::NU; ++j) {
            const int u = tid + kThreads * j;
            if (u < total) {
                if (u < 2 * F::UQ) {
                    const int x = u < F::UQ ? u : u - F::UQ;
                    const int tb = x / (F::KS / 8), db = x % (F::KS / 8);
                    const int pair0 = (sl * F::KS + db * 8) / 2;
                    const long long p0 = a.pos0 + t0 + tb * 8;
                    if (u < F::UQ)
                        commit_q<E>(buf[j], L - tb * 8, a.rotate, a.theta, pair0, p0, sQ + tb * 8 * F::LDQ + db * 8,
                                    F::LDQ);
                    else
                        commit_k<E>(buf[j], L - tb * 8, a.rotate, a.theta, pair0, p0, lg, L - 1 - tb * 8,
                                    sK + tb * 8 * F::LDQ + db * 8, F::LDQ, sKc + db * 8 * F::LDC + tb * 8, F::LDC);
                } else {
                    const int x = u - 2 * F::UQ;
                    const int tb = x / (DVT / 8), db = x % (DVT / 8);
                    commit_v(buf[j], L - tb * 8, sVc + db * 8 * F::LDC + tb * 8, F::LDC);
                }
            }
        }
    };

    f32x4_t S[F::NS_W], O[F::NO_W];
    if (nst > 0) issue(0);
    for (int i = 0; i < nst; ++i) {
        const int sl = i % F::NSL;
        const long long t0 = seg_t0 + (long long)(i / F::NSL) * C;
        const int L = (int)min((long long)C, seg_t1 - t0);
        if (sl == 0) {
#pragma unroll
            for (int x = 0; x < F::NS_W; ++x) S[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int x = 0; x < F::NO_W; ++x) O[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();  // staging buffers free; previous copies of R and of the output tile consumed
        commit(i);
        if (i + 1 < nst) issue(i + 1);
        __syncthreads();
        // S += Q_s K_s^T over the lower-triangle tiles.
#pragma unroll
        for (int rb = 0, t = 0; rb < F::NB; ++rb)
#pragma unroll
            for (int cb = 0; cb <= rb; ++cb, ++t)
                if (t % kWaves == w)
                    mma_nt(S[t / kWaves], sQ + rb * 16 * F::LDQ, F::LDQ, sK + cb * 16 * F::LDQ, F::LDQ, F::KS, lane);
        // O += Q_s R_s (cross-chunk read of the state carried in from the previous chunk).
#pragma unroll
        for (int x = 0; x < F::NO_W; ++x) {
            const int t = w + kWaves * x;
            if (t < F::NO) {
                const int rb = t / F::NDV, cb = t % F::NDV;
                mma_nt(O[x], sQ + rb * 16 * F::LDQ, F::LDQ, sRt + cb * 16 * F::LDR + sl * F::KS, F::LDR, F::KS, lane);
            }
        }
        // R_s <- gamma^L R_s + K_s^T (V (.) zeta): zeta is folded into sKc.
        const float gL = gpow(lg, (float)L);
#pragma unroll
        for (int x = 0; x < F::NR_W; ++x) {
            const int t = w + kWaves * x;
            const int rb = t / F::NDV, cb = t % F::NDV;
            if (t < F::NR && rb / (F::KS / 16) == sl) {
                R[x] *= gL;
                mma_nt(R[x], sKc + (rb - sl * (F::KS / 16)) * 16 * F::LDC, F::LDC, sVc + cb * 16 * F::LDC, F::LDC, C,
                       lane);
            }
        }
        if (sl != F::NSL - 1) continue;

        // Decay mask in registers: P[j][l] = S[j][l] * gamma^(j-l) for l <= j.
#pragma unroll
        for (int rb = 0, t = 0; rb < F::NB; ++rb)
#pragma unroll
            for (int cb = 0; cb <= rb; ++cb, ++t)
                if (t % kWaves == w) {
                    const int l = cb * 16 + (lane & 15);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = rb * 16 + 4 * (lane >> 4) + e;
                        const float val = (l <= j) ? S[t / kWaves][e] * gpow(lg, (float)(j - l)) : 0.f;
                        if constexpr (sizeof(st) == 2)
                            sP[j * F::LDC + l] = f32_to_bf16(val);
                        else
                            sP[j * F::LDC + l] = val;
                    }
                }
        __syncthreads();  // P complete; all reads of sQ/sK/sRt for this chunk are done
        // O = (Q R) (.) xi + P V, written to the output tile in LDS.
#pragma unroll
        for (int x = 0; x < F::NO_W; ++x) {
            const int t = w + kWaves * x;
            if (t < F::NO) {
                const int rb = t / F::NDV, cb = t % F::NDV;
#pragma unroll
                for (int e = 0; e < 4; ++e) O[x][e] *= gpow(lg, (float)(rb * 16 + 4 * (lane >> 4) + e + 1));
                const int kmax = min(C, ((rb + 1) * 16 + E::KD - 1) / E::KD * E::KD);
                mma_nt(O[x], sP + rb * 16 * F::LDC, F::LDC, sVc + cb * 16 * F::LDC, F::LDC, kmax, lane);
                const int col = cb * 16 + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = rb * 16 + 4 * (lane >> 4) + e;
                    if (a.out_bf16)
                        reinterpret_cast<uint16_t*>(sO)[j * F::LDO + col] = f32_to_bf16(O[x][e]);
                    else
                        reinterpret_cast<float*>(sO)[j * F::LDO + col] = O[x][e];
                }
            }
        }
        // New operand copy of R for the next chunk.
#pragma unroll
        for (int x = 0; x < F::NR_W; ++x) {
            const int t = w + kWaves * x;
            if (t < F::NR) {
                const int rb = t / F::NDV, cb = t % F::NDV;
                store4(sRt + (cb * 16 + (lane & 15)) * F::LDR + rb * 16 + 4 * (lane >> 4), R[x]);
            }
        }
        __syncthreads();
        // Coalesced 16-byte stores of the output rows j < L.
        const int vec = 16 / osz;                  // elements per 16-byte store
        const int per_row = DVT / vec;
        char* obase = (char*)a.o + ((qk_row0 + t0 * a.H) * a.dv + dv0) * osz;
        for (int x = tid; x < L * per_row; x += kThreads) {
            const int j = x / per_row, c16 = x % per_row;
            *reinterpret_cast<uint4*>(obase + ((long long)j * a.H * a.dv + c16 * vec) * osz) =
                *reinterpret_cast<const uint4*>(sO + (j * F::LDO + c16 * vec) * osz);
        }
    }
    // The state after the last token of the sequence.
    if (seg == a.nseg - 1 && a.state_out) {
        float* out = a.state_out + (long long)pair * DK * a.dv;
#pragma unroll
        for (int i = 0; i < F::NR_W; ++i) {
            const int t = w + kWaves * i;
            if (t < F::NR) {
                const int rb = t / F::NDV, cb = t % F::NDV;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    out[(long long)(rb * 16 + 4 * (lane >> 4) + e) * a.dv + dv0 + cb * 16 + (lane & 15)] = R[i][e];
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------------
// chunk_local: end state of segment g from a zero state, written to workspace slot g + 1 (g < nseg - 1).
// ---------------------------------------------------------------------------------------------------
template <class E, int DK, int C, int DVT>
struct LocalCfg {
    typedef typename E::st st;
    static constexpr int LDC = C + E::PAD;
    static constexpr int NDV = DVT / 16, NKB = DK / 16;
    static constexpr int NR = NKB * NDV;
    static constexpr int NR_W = (NR + kWaves - 1) / kWaves;
    static constexpr int UK = (C / 8) * (DK / 8), UV = (C / 8) * (DVT / 8);
    static constexpr int NU = (UK + UV + kThreads - 1) / kThreads;
    static constexpr int SKC = DK * LDC, SVC = DVT * LDC;
    static constexpr int LDS_BYTES = (SKC + SVC) * (int)sizeof(st);
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <class E, int DK, int C, int DVT>
__global__ __launch_bounds__(kThreads, 2) void chunk_local_kernel(FwdArgs a) {
    typedef LocalCfg<E, DK, C, DVT> F;
    typedef typename E::st st;
    __shared__ __attribute__((aligned(16))) st smem[F::LDS_BYTES / sizeof(st)];
    st* sKc = smem;
    st* sVc = smem + F::SKC;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int seg = blockIdx.x, dvt = blockIdx.y, pair = blockIdx.z;
    const Seq s{a.N, a.H, pair / a.H, pair % a.H};
    const int dv0 = dvt * DVT;
    const float lg = a.log2g[s.h];
    const st* k = (const st*)a.k;
    const st* v = (const st*)a.v;

    f32x4_t R[F::NR_W];
#pragma unroll
    for (int i = 0; i < F::NR_W; ++i) R[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const long long seg_t0 = (long long)seg * a.seg_len;
    const long long seg_t1 = min((long long)a.N, seg_t0 + a.seg_len);
    const int nst = (int)((seg_t1 - seg_t0 + C - 1) / C);
    const long long row0 = ((long long)s.b * a.N) * a.H + s.h;
    const int rsk = a.H * a.dk, rsv = a.H * a.dv;

    Raw<E> buf[F::NU];
    auto issue = [&](int i) {
        const long long t0 = seg_t0 + (long long)i * C;
        const int L = (int)min((long long)C, seg_t1 - t0);
#pragma unroll
        for (int j = 0; j < F::NU; ++j) {
            const int u = tid + kThreads * j;
            if (u < F::UK + F::UV) {
                if (u < F::UK) {
                    const int tb = u / (DK / 8);
                    issue_unit(buf[j], k + (row0 + (t0 + tb * 8) * a.H) * a.dk + (u % (DK / 8)) * 8, rsk, L - tb * 8);
                } else {
                    const int x = u - F::UK, tb = x / (DVT / 8);
                    issue_unit(buf[j], v + (row0 + (t0 + tb * 8) * a.H) * a.dv + dv0 + (x % (DVT / 8)) * 8, rsv,
                               L - tb * 8);
                }
            }
        }
    };
    auto commit = [&](int i) {
        const long long t0 = seg_t0 + (long long)i * C;
        const int L = (int)min((long long)C, seg_t1 - t0);
#pragma unroll
        for (int j = 0; j < F::NU; ++j) {
            const int u = tid + kThreads * j;
            if (u < F::UK + F::UV) {
                if (u < F::UK) {
                    const int tb = u / (DK / 8), db = u % (DK / 8);
                    commit_k<E>(buf[j], L - tb * 8, a.rotate, a.theta, db * 4, a.pos0 + t0 + tb * 8, lg, L - 1 - tb * 8,
                                nullptr, 0, sKc + db * 8 * F::LDC + tb * 8, F::LDC);
                } else {
                    const int x = u - F::UK, tb = x / (DVT / 8), db = x % (DVT / 8);
                    commit_v(buf[j], L - tb * 8, sVc + db * 8 * F::LDC + tb * 8, F::LDC);
                }
            }
        }
    };

    if (nst > 0) issue(0);
    for (int i = 0; i < nst; ++i) {
        const long long t0 = seg_t0 + (long long)i * C;
        const int L = (int)min((long long)C, seg_t1 - t0);
        __syncthreads();
        commit(i);
        if (i + 1 < nst) issue(i + 1);
        __syncthreads();
        const float gL = gpow(lg, (float)L);
#pragma unroll
        for (int x = 0; x < F::NR_W; ++x) {
            const int t = w + kWaves * x;
            if (t < F::NR) {
                const int rb = t / F::NDV, cb = t % F::NDV;
                R[x] *= gL;
                mma_nt(R[x], sKc + rb * 16 * F::LDC, F::LDC, sVc + cb * 16 * F::LDC, F::LDC, C, lane);
            }
        }
    }
    float* out = a.ws + ((long long)pair * a.nseg + seg + 1) * DK * a.dv;
#pragma unroll
    for (int i = 0; i < F::NR_W; ++i) {
        const int t = w + kWaves * i;
        if (t < F::NR) {
            const int rb = t / F::NDV, cb = t % F::NDV;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[(long long)(rb * 16 + 4 * (lane >> 4) + e) * a.dv + dv0 + cb * 16 + (lane & 15)] = R[i][e];
        }
    }
}

// ---------------------------------------------------------------------------------------------------
// parallel_fwd: one workgroup per (query block, d_v tile, b*H + h); key blocks 0..qb.
// ---------------------------------------------------------------------------------------------------
template <class E, int DK, int BQ, int DVT>
struct ParCfg {
    typedef typename E::st st;
    static constexpr int LDQ = DK + E::PAD, LDC = BQ + E::PAD;
    static constexpr int NB = BQ / 16, NDV = DVT / 16;
    static constexpr int NSQ = NB * NB, NS_W = (NSQ + kWaves - 1) / kWaves;
    static constexpr int NO = NB * NDV, NO_W = (NO + kWaves - 1) / kWaves;
    static constexpr int SQ = BQ * LDQ, SVC = DVT * LDC, SP = BQ * LDC;
    static constexpr int LDS_BYTES = (2 * SQ + SVC + SP) * (int)sizeof(st);
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <class E, int DK, int BQ, int DVT>
__global__ __launch_bounds__(kThreads, 2) void parallel_kernel(FwdArgs a) {
    typedef ParCfg<E, DK, BQ, DVT> F;
    typedef typename E::st st;
    __shared__ __attribute__((aligned(16))) st smem[F::LDS_BYTES / sizeof(st)];
    st* sQ = smem;
    st* sK = sQ + F::SQ;
    st* sVc = sK + F::SQ;
    st* sP = sVc + F::SVC;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int qb = blockIdx.x, dvt = blockIdx.y, pair = blockIdx.z;
    const Seq s{a.N, a.H, pair / a.H, pair % a.H};
    const int dv0 = dvt * DVT;
    const float lg = a.log2g[s.h];
    const long long q0 = (long long)qb * BQ;
    const int LQ = (int)min((long long)BQ, a.N - q0);

    stage_qk<E, BQ, DK, true, false, false>((const st*)a.q, (const st*)a.q, s, a.dk, q0, LQ, 0, a.theta, a.rotate, a.pos0, lg, sQ, F::LDQ,
                        nullptr, 0, nullptr, 0, tid);
    f32x4_t O[F::NO_W];
#pragma unroll
    for (int i = 0; i < F::NO_W; ++i) O[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int kb = 0; kb <= qb; ++kb) {
        const long long k0 = (long long)kb * BQ;
        const int LK = (int)min((long long)BQ, a.N - k0);
        __syncthreads();
        stage_qk<E, BQ, DK, false, true, false>((const st*)a.k, (const st*)a.k, s, a.dk, k0, LK, 0, a.theta, a.rotate, a.pos0, lg,
                            nullptr, 0, sK, F::LDQ, nullptr, 0, tid);
        stage_v<E, BQ, DVT>((const st*)a.v, s, a.dv, k0, LK, dv0, sVc, F::LDC, tid);
        __syncthreads();
        f32x4_t S[F::NS_W];
#pragma unroll
        for (int i = 0; i < F::NS_W; ++i) {
            const int t = w + kWaves * i;
            S[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (t < F::NSQ) {
                const int rb = t / F::NB, cb = t % F::NB;
                mma_nt(S[i], sQ + rb * 16 * F::LDQ, F::LDQ, sK + cb * 16 * F::LDQ, F::LDQ, DK, lane);
                const int l = cb * 16 + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = rb * 16 + 4 * (lane >> 4) + e;
                    const long long dist = (q0 + j) - (k0 + l);  // n - m
                    const float val = (dist >= 0) ? S[i][e] * gpow(lg, (float)dist) : 0.f;
                    if constexpr (sizeof(st) == 2)
                        sP[j * F::LDC + l] = f32_to_bf16(val);
                    else
                        sP[j * F::LDC + l] = val;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < F::NO_W; ++i) {
            const int t = w + kWaves * i;
            if (t < F::NO) {
                const int rb = t / F::NDV, cb = t % F::NDV;
                mma_nt(O[i], sP + rb * 16 * F::LDC, F::LDC, sVc + cb * 16 * F::LDC, F::LDC, BQ, lane);
            }
        }
    }
    const long long obase = ((long long)s.b * a.N + q0) * a.H + s.h;
#pragma unroll
    for (int i = 0; i < F::NO_W; ++i) {
        const int t = w + kWaves * i;
        if (t < F::NO) {
            const int rb = t / F::NDV, cb = t % F::NDV;
            const int col = dv0 + cb * 16 + (lane & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = rb * 16 + 4 * (lane >> 4) + e;
                if (j < LQ) {
                    const long long off = (obase + (long long)j * a.H) * a.dv + col;
                    if (a.out_bf16)
                        store_out((uint16_t*)a.o + off, O[i][e]);
                    else
                        store_out((float*)a.o + off, O[i][e]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------------
// recurrent_step: one workgroup per (64-column d_v tile, b*H + h). Thread (rg, cg): columns 4cg..4cg+3 of the
// tile, rows rg, rg+16, ... Each row update S = gamma S + k_r v is a float4 read-modify-write; the partial
// sums of o = q S are reduced over the 16 row groups in LDS.
// ---------------------------------------------------------------------------------------------------
struct StepArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* state;
    int B, H, dk, dv;
    int in_bf16, out_bf16, rotate;
    long long pos;
    float gamma[kMaxHeads];
    double theta[kMaxPairs];
};

__device__ __forceinline__ float ld_in(const void* p, long long i, int bf) {
    return bf ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

template <int DK>
__global__ __launch_bounds__(kThreads) void recurrent_step_kernel(StepArgs a) {
    __shared__ float sq[DK], sk[DK];
    __shared__ float4 part[16][16];
    const int tid = threadIdx.x, cg = tid & 15, rg = tid >> 4;
    const int pair = blockIdx.y, h = pair % a.H;
    const int c0 = blockIdx.x * 64 + 4 * cg;
    const long long qk0 = (long long)pair * a.dk;
    // Rotated q and k (fp32) for this head and position.
    for (int i = tid; i < a.dk / 2; i += kThreads) {
        float q0 = ld_in(a.q, qk0 + 2 * i, a.in_bf16), q1 = ld_in(a.q, qk0 + 2 * i + 1, a.in_bf16);
        float k0 = ld_in(a.k, qk0 + 2 * i, a.in_bf16), k1 = ld_in(a.k, qk0 + 2 * i + 1, a.in_bf16);
        if (a.rotate) {
            float c, sn;
            rot_cs(a.pos, a.theta[i], &c, &sn);
            sq[2 * i] = q0 * c - q1 * sn;
            sq[2 * i + 1] = q0 * sn + q1 * c;
            sk[2 * i] = k0 * c - k1 * sn;
            sk[2 * i + 1] = k0 * sn + k1 * c;
        } else {
            sq[2 * i] = q0;
            sq[2 * i + 1] = q1;
            sk[2 * i] = k0;
            sk[2 * i + 1] = k1;
        }
    }
    const bool active = c0 < a.dv;
    float4 vv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (active) {
        const long long vo = (long long)pair * a.dv + c0;
        vv = make_float4(ld_in(a.v, vo, a.in_bf16), ld_in(a.v, vo + 1, a.in_bf16), ld_in(a.v, vo + 2, a.in_bf16),
                         ld_in(a.v, vo + 3, a.in_bf16));
    }
    __syncthreads();
    const float g = a.gamma[h];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (active) {
        constexpr int RPT = DK / 16;  // rows per thread
        float* S = a.state + (long long)pair * DK * a.dv + c0;
        float4 x[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) x[i] = *reinterpret_cast<const float4*>(S + (long long)(rg + 16 * i) * a.dv);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + 16 * i;
            const float kr = sk[r], qr = sq[r];
            x[i].x = g * x[i].x + kr * vv.x;
            x[i].y = g * x[i].y + kr * vv.y;
            x[i].z = g * x[i].z + kr * vv.z;
            x[i].w = g * x[i].w + kr * vv.w;
            acc.x += qr * x[i].x;
            acc.y += qr * x[i].y;
            acc.z += qr * x[i].z;
            acc.w += qr * x[i].w;
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) *reinterpret_cast<float4*>(S + (long long)(rg + 16 * i) * a.dv) = x[i];
    }
    part[rg][cg] = acc;
    __syncthreads();
    if (tid < 64) {
        const int cgo = tid >> 2, comp = tid & 3;
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float4 p = part[r][cgo];
            sum += comp == 0 ? p.x : comp == 1 ? p.y : comp == 2 ? p.z : p.w;
        }
        const int col = blockIdx.x * 64 + tid;
        if (col < a.dv) {
            const long long off = (long long)pair * a.dv + col;
            if (a.out_bf16)
                store_out((uint16_t*)a.o + off, sum);
            else
                store_out((float*)a.o + off, sum);
        }
    }
}

}  // namespace ret


namespace ret {

typedef void (*fwd_kernel_t)(FwdArgs);
typedef void (*step_kernel_t)(StepArgs);

struct ChunkKernels {
    fwd_kernel_t full, local;
    int dvt;
};
struct ParKernel {
    fwd_kernel_t fn;
    int bq, dvt;
};

template <class E, int DK, int C, int DVT>
ChunkKernels chunk_entry() {
    return {chunk_full_kernel<E, DK, C, DVT>, chunk_local_kernel<E, DK, C, DVT>, DVT};
}

// Getters, one per kernel-group source. Return false when the shape has no instance.
bool chunk_kernels_f32(int dk, int dv, int C, ChunkKernels* out);
bool chunk_kernels_bf16_small(int dk, int dv, int C, ChunkKernels* out);   // d_k in {32, 64}
bool chunk_kernels_bf16_128(int dk, int dv, int C, ChunkKernels* out);     // d_k = 128
bool chunk_kernels_bf16_256(int dk, int dv, int C, ChunkKernels* out);     // d_k = 256
bool parallel_kernel_get(bool bf16_in, int dk, int dv, ParKernel* out);
step_kernel_t step_kernel_get(int dk);
fwd_kernel_t segment_scan_get();

}  // namespace ret
