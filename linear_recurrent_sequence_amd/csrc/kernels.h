// Kernel templates of libretention.so (gfx950). Each kernel-group source instantiates a subset and exposes
// getters; the C-ABI source launches them.
#pragma once

#include <type_traits>

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

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0..N-1.
template <int I, int N, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Tile t of the lower triangle (lb <= jb), enumerated row by row, as (jb, lb). t is wave-uniform, so this
// runs on the scalar unit.
template <int NB>
__device__ __forceinline__ void tri_tile(int t, int& jb, int& lb) {
    int r = 0;
#pragma unroll
    for (int i = 1; i < NB; ++i) r += (t >= i * (i + 1) / 2) ? 1 : 0;
    jb = r;
    lb = t - r * (r + 1) / 2;
}

// ---------------------------------------------------------------------------------------------------
// chunk_full: one workgroup per (segment, d_v tile, b*H + h). The segment's chunks are processed in stages
// (chunk, d_k slice); the global loads of stage i+1 are issued before stage i is computed.
// Products are formed transposed where that helps the stores: S^T = K Q^T (each lane then holds 4 consecutive
// keys of one query row of P) and O^T = R^T Q^T + V^T P^T (4 consecutive d_v of one output row).
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
    typedef ItemWidth<C, KS> IQK;                    // Q+K staging items per slice
    typedef ItemWidth<C, DVT> IV;                    // V staging items (first slice only)
    static constexpr int SQ = C * LDQ, SKC = KS * LDC, SVC = DVT * LDC, SP = C * LDC, SRT = DVT * LDR;
    // Region A holds sQ, sK and sKc while a chunk's slices are computed, then the output tile (fp32 at most).
    static constexpr int A_STAGE = (2 * SQ + SKC) * (int)sizeof(st), A_OUT = C * LDO * 4;
    static constexpr int A_BYTES = ((A_STAGE > A_OUT ? A_STAGE : A_OUT) + 15) / 16 * 16;
    static constexpr int LDS_BYTES = A_BYTES + (SVC + SP + SRT) * (int)sizeof(st);
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(C % 16 == 0 && DVT % 16 == 0 && DK % KS == 0 && KS % E::KD == 0 && C % E::KD == 0, "tiling");
};

// O^T tile x of wave w covers query block jb and d_v block db; with four d_v blocks, jb = x and db = w.
template <class F>
__device__ __forceinline__ int ojb(int w, int x) {
    return F::NDV == kWaves ? x : (w + kWaves * x) / F::NDV;
}
template <class F>
__device__ __forceinline__ int odb(int w, int x) {
    return F::NDV == kWaves ? w : (w + kWaves * x) % F::NDV;
}

template <class E, int DK, int C, int DVT>
__global__ __launch_bounds__(kThreads, 2) void chunk_full_kernel(FwdArgs a) {
    typedef FullCfg<E, DK, C, DVT> F;
    typedef typename E::st st;
    constexpr int IQ = F::IQK::value, IVW = F::IV::value, NIQ = F::IQK::per_thread, NIV = F::IV::per_thread;
    __shared__ __attribute__((aligned(16))) st smem[F::LDS_BYTES / sizeof(st)];
    st* sQ = smem;
    st* sK = sQ + F::SQ;
    st* sKc = sK + F::SQ;
    st* sVc = smem + F::A_BYTES / sizeof(st);
    st* sP = sVc + F::SVC;
    st* sRt = sP + F::SP;
    char* sO = reinterpret_cast<char*>(smem);  // output tile, over region A once a chunk's slices are done

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g4 = 4 * (lane >> 4), n16 = lane & 15;
    const int seg = blockIdx.x, dvt = blockIdx.y, pair = blockIdx.z;
    const int b = pair / a.H, h = pair % a.H;
    const int dv0 = dvt * DVT;
    const float lg = a.log2g[h];
    const int osz = a.out_bf16 ? 2 : 4;

    // Scores above the diagonal are never written: keep them zero for the P.V product.
    for (int i = tid; i < F::SP; i += kThreads) sP[i] = (st)0;

    // Decay factors that do not depend on the chunk: the mask gamma^(j-l) of each owned S^T tile (rows l,
    // columns j) and xi_j = gamma^(j+1) of each owned O^T tile (columns j).
    // S^T tiles of this wave: t = w + 4x in row-by-row lower-triangle order.
    int Sjb[F::NS_W], Slb[F::NS_W];
    float Dm[F::NS_W][4], Xi[F::NO_W];
#pragma unroll
    for (int x = 0; x < F::NS_W; ++x) {
        tri_tile<F::NB>(min(w + kWaves * x, F::NS - 1), Sjb[x], Slb[x]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int d = 16 * (Sjb[x] - Slb[x]) + n16 - g4 - e;  // j - l
            Dm[x][e] = d >= 0 ? gpow(lg, (float)d) : 0.f;
        }
    }
#pragma unroll
    for (int x = 0; x < F::NO_W; ++x) Xi[x] = gpow(lg, (float)(ojb<F>(w, x) * 16 + n16 + 1));

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
            for (int e = 0; e < 4; ++e) R[i][e] = init[(long long)(rb * 16 + g4 + e) * a.dv + dv0 + cb * 16 + n16];
        }
    }
    // Copy of R (operand precision), transposed to [d_v][d_k], for the cross product.
#pragma unroll
    for (int i = 0; i < F::NR_W; ++i) {
        const int t = w + kWaves * i;
        if (t < F::NR) {
            const int rb = t / F::NDV, cb = t % F::NDV;
            store4(sRt + (cb * 16 + n16) * F::LDR + rb * 16 + g4, R[i]);
        }
    }

    const long long seg_t0 = (long long)seg * a.seg_len;
    const long long seg_t1 = min((long long)a.N, seg_t0 + a.seg_len);
    const int nst = (int)((seg_t1 - seg_t0 + C - 1) / C) * F::NSL;
    const int rsk = a.H * a.dk, rsv = a.H * a.dv;
    // This thread's staging items: token block and first dim; pointers at the segment's first chunk.
    int qtb[NIQ], qdb[NIQ], vtb[NIV], vdb[NIV];
    const st *qp[NIQ], *kp[NIQ], *vp[NIV];
    RotStep<IQ / 2> rstep[NIQ][F::NSL];
    float zfull[NIQ][8];
#pragma unroll
    for (int j = 0; j < NIQ; ++j) {
        const int x = min(tid + kThreads * j, F::IQK::count - 1);
        qtb[j] = x / (F::KS / IQ);
        qdb[j] = x % (F::KS / IQ);
        const long long off = (((long long)b * a.N + seg_t0 + qtb[j] * 8) * a.H + h) * a.dk + qdb[j] * IQ;
        qp[j] = (const st*)a.q + off;
        kp[j] = (const st*)a.k + off;
#pragma unroll
        for (int sl = 0; sl < F::NSL; ++sl)
            if (a.rotate) rstep[j][sl].init(a.theta, (sl * F::KS + qdb[j] * IQ) / 2);
        item_zeta(zfull[j], lg, C - 1 - qtb[j] * 8, 8);
    }
#pragma unroll
    for (int j = 0; j < NIV; ++j) {
        const int x = min(tid + kThreads * j, F::IV::count - 1);
        vtb[j] = x / (DVT / IVW);
        vdb[j] = x % (DVT / IVW);
        vp[j] = (const st*)a.v + (((long long)b * a.N + seg_t0 + vtb[j] * 8) * a.H + h) * a.dv + dv0 + vdb[j] * IVW;
    }
    const float gC = gpow(lg, (float)C);

    Item<E, IQ> bq[NIQ], bk[NIQ];
    Item<E, IVW> bv[NIV];
    auto issue = [&](int i) {
        const int c = i / F::NSL, sl = i % F::NSL;
        const int L = (int)min((long long)C, seg_t1 - seg_t0 - (long long)c * C);
        const long long cq = (long long)c * C * rsk + sl * F::KS;
#pragma unroll
        for (int j = 0; j < NIQ; ++j)
            if (tid + kThreads * j < F::IQK::count) {
                issue_item<E, IQ>(bq[j], qp[j] + cq, rsk, L - qtb[j] * 8);
                issue_item<E, IQ>(bk[j], kp[j] + cq, rsk, L - qtb[j] * 8);
            }
        if (sl == 0) {
            const long long cv = (long long)c * C * rsv;
#pragma unroll
            for (int j = 0; j < NIV; ++j)
                if (tid + kThreads * j < F::IV::count) issue_item<E, IVW>(bv[j], vp[j] + cv, rsv, L - vtb[j] * 8);
        }
    };
    auto commit = [&](int i) {
        const int c = i / F::NSL, sl = i % F::NSL;
        const long long t0 = seg_t0 + (long long)c * C;
        const int L = (int)min((long long)C, seg_t1 - t0);
#pragma unroll
        for (int j = 0; j < NIQ; ++j)
            if (tid + kThreads * j < F::IQK::count) {
                float zt[8];
                if (L == C) {
#pragma unroll
                    for (int r = 0; r < 8; ++r) zt[r] = zfull[j][r];
                } else {
                    item_zeta(zt, lg, L - 1 - qtb[j] * 8, L - qtb[j] * 8);
                }
                RotStep<IQ / 2> rs = rstep[j][0];
#pragma unroll
                for (int x = 1; x < F::NSL; ++x)
                    if (sl == x) rs = rstep[j][x];
                commit_qk<E, IQ, true, true>(&bq[j], bk[j], L - qtb[j] * 8, a.rotate, a.theta,
                                             (sl * F::KS + qdb[j] * IQ) / 2, a.pos0 + t0 + qtb[j] * 8, rs, zt,
                                             sQ + qtb[j] * 8 * F::LDQ + qdb[j] * IQ, F::LDQ,
                                             sK + qtb[j] * 8 * F::LDQ + qdb[j] * IQ, F::LDQ,
                                             sKc + qdb[j] * IQ * F::LDC + qtb[j] * 8, F::LDC);
            }
        if (sl == 0) {
#pragma unroll
            for (int j = 0; j < NIV; ++j)
                if (tid + kThreads * j < F::IV::count)
                    commit_vcol<E, IVW>(bv[j], L - vtb[j] * 8, sVc + vdb[j] * IVW * F::LDC + vtb[j] * 8, F::LDC);
        }
    };

    const int nchunks = nst / F::NSL;
    if (nst > 0) issue(0);
    for (int c = 0; c < nchunks; ++c) {
        const long long t0 = seg_t0 + (long long)c * C;
        const int L = (int)min((long long)C, seg_t1 - t0);
        const float gL = L == C ? gC : gpow(lg, (float)L);
        f32x4_t S[F::NS_W], O[F::NO_W];
#pragma unroll
        for (int x = 0; x < F::NS_W; ++x) S[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int x = 0; x < F::NO_W; ++x) O[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        static_for<0, F::NSL>([&](auto slc) {
            constexpr int sl = decltype(slc)::value;
            const int i = c * F::NSL + sl;
            __syncthreads();  // staging buffers free; previous copies of R and of the output tile consumed
            commit(i);
            if (i + 1 < nst) issue(i + 1);
            __syncthreads();
            // S^T += K_s Q_s^T over this wave's lower-triangle tiles (keys l <= queries j). Slots past the last
            // tile repeat it; their results are never stored.
#pragma unroll
            for (int x = 0; x < F::NS_W; ++x)
                mma_nt(S[x], sK + Slb[x] * 16 * F::LDQ, F::LDQ, sQ + Sjb[x] * 16 * F::LDQ, F::LDQ, F::KS, lane);
            // O^T += R_s^T Q_s^T (cross-chunk read of the state carried in from the previous chunk).
#pragma unroll
            for (int x = 0; x < F::NO_W; ++x)
                if (F::NO % kWaves == 0 || w + kWaves * x < F::NO) {
                    const int jb = ojb<F>(w, x), db = odb<F>(w, x);
                    mma_nt(O[x], sRt + db * 16 * F::LDR + sl * F::KS, F::LDR, sQ + jb * 16 * F::LDQ, F::LDQ, F::KS,
                           lane);
                }
            // R_s <- gamma^L R_s + K_s^T (V (.) zeta): zeta is folded into sKc. R tile x of wave w covers d_k
            // block rb = (w + 4x) / NDV; with four d_v blocks rb = x, known at compile time.
#pragma unroll
            for (int x = 0; x < F::NR_W; ++x) {
                const int t = w + kWaves * x;
                const int rb = F::NDV == kWaves ? x : t / F::NDV, cb = F::NDV == kWaves ? w : t % F::NDV;
                if ((F::NR % kWaves == 0 || t < F::NR) && rb / (F::KS / 16) == sl) {
                    R[x] *= gL;
                    mma_nt(R[x], sKc + (rb - sl * (F::KS / 16)) * 16 * F::LDC, F::LDC, sVc + cb * 16 * F::LDC,
                           F::LDC, C, lane);
                }
            }
        });

        // Decay mask: P[j][l..l+3] = S^T[l..l+3][j] * gamma^(j-l), four consecutive keys per store.
#pragma unroll
        for (int x = 0; x < F::NS_W; ++x)
            if (w + kWaves * x < F::NS) {
                f32x4_t pv;
#pragma unroll
                for (int e = 0; e < 4; ++e) pv[e] = S[x][e] * Dm[x][e];
                store4(sP + (Sjb[x] * 16 + n16) * F::LDC + Slb[x] * 16 + g4, pv);
            }
        __syncthreads();  // P complete; all reads of sQ/sK/sKc/sRt for this chunk are done
        // O^T = xi (.) (R^T Q^T) + V^T P^T, then the output tile in LDS (4 consecutive d_v per store).
#pragma unroll
        for (int x = 0; x < F::NO_W; ++x) {
            if (F::NO % kWaves == 0 || w + kWaves * x < F::NO) {
                const int jb = ojb<F>(w, x), db = odb<F>(w, x);
                O[x] *= Xi[x];
                const int kmax = min(C, ((jb + 1) * 16 + E::KD - 1) / E::KD * E::KD);
                mma_nt(O[x], sVc + db * 16 * F::LDC, F::LDC, sP + jb * 16 * F::LDC, F::LDC, kmax, lane);
                const int row = jb * 16 + n16, col = db * 16 + g4;
                if (a.out_bf16)
                    store4(reinterpret_cast<uint16_t*>(sO) + row * F::LDO + col, O[x]);
                else
                    store4(reinterpret_cast<float*>(sO) + row * F::LDO + col, O[x]);
            }
        }
        // New operand copy of R for the next chunk.
#pragma unroll
        for (int x = 0; x < F::NR_W; ++x) {
            const int t = w + kWaves * x;
            if (F::NR % kWaves == 0 || t < F::NR) {
                const int rb = F::NDV == kWaves ? x : t / F::NDV, cb = F::NDV == kWaves ? w : t % F::NDV;
                store4(sRt + (cb * 16 + n16) * F::LDR + rb * 16 + g4, R[x]);
            }
        }
        __syncthreads();
        // Coalesced 16-byte stores of the output rows j < L.
        const int vec = 16 / osz;  // elements per 16-byte store
        const int per_row = DVT / vec;
        char* obase = (char*)a.o + ((((long long)b * a.N + t0) * a.H + h) * a.dv + dv0) * osz;
        for (int x = tid; x < L * per_row; x += kThreads) {
            const int j = x / per_row, c16 = x % per_row;
            *reinterpret_cast<uint4*>(obase + ((long long)j * rsv + c16 * vec) * osz) =
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
                for (int e = 0; e < 4; ++e) out[(long long)(rb * 16 + g4 + e) * a.dv + dv0 + cb * 16 + n16] = R[i][e];
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
    typedef ItemWidth<C, DK> IK;
    typedef ItemWidth<C, DVT> IV;
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

    constexpr int IKW = F::IK::value, IVW = F::IV::value;
    Item<E, IKW> bk[F::IK::per_thread];
    Item<E, IVW> bv[F::IV::per_thread];
    auto issue = [&](int i) {
        const long long t0 = seg_t0 + (long long)i * C;
        const int L = (int)min((long long)C, seg_t1 - t0);
#pragma unroll
        for (int j = 0; j < F::IK::per_thread; ++j) {
            const int x = tid + kThreads * j;
            if (x < F::IK::count) {
                const int tb = x / (DK / IKW), db = x % (DK / IKW);
                issue_item<E, IKW>(bk[j], k + (row0 + (t0 + tb * 8) * a.H) * a.dk + db * IKW, rsk, L - tb * 8);
            }
        }
#pragma unroll
        for (int j = 0; j < F::IV::per_thread; ++j) {
            const int x = tid + kThreads * j;
            if (x < F::IV::count) {
                const int tb = x / (DVT / IVW), db = x % (DVT / IVW);
                issue_item<E, IVW>(bv[j], v + (row0 + (t0 + tb * 8) * a.H) * a.dv + dv0 + db * IVW, rsv, L - tb * 8);
            }
        }
    };
    auto commit = [&](int i) {
        const long long t0 = seg_t0 + (long long)i * C;
        const int L = (int)min((long long)C, seg_t1 - t0);
#pragma unroll
        for (int j = 0; j < F::IK::per_thread; ++j) {
            const int x = tid + kThreads * j;
            if (x < F::IK::count) {
                const int tb = x / (DK / IKW), db = x % (DK / IKW);
                float zt[8];
                item_zeta(zt, lg, L - 1 - tb * 8, L - tb * 8);
                RotStep<IKW / 2> rs;
                if (a.rotate) rs.init(a.theta, db * IKW / 2);
                commit_qk<E, IKW, false, false>(nullptr, bk[j], L - tb * 8, a.rotate, a.theta, db * IKW / 2,
                                                a.pos0 + t0 + tb * 8, rs, zt, nullptr, 0, nullptr, 0,
                                                sKc + db * IKW * F::LDC + tb * 8, F::LDC);
            }
        }
#pragma unroll
        for (int j = 0; j < F::IV::per_thread; ++j) {
            const int x = tid + kThreads * j;
            if (x < F::IV::count) {
                const int tb = x / (DVT / IVW), db = x % (DVT / IVW);
                commit_vcol<E, IVW>(bv[j], L - tb * 8, sVc + db * IVW * F::LDC + tb * 8, F::LDC);
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
