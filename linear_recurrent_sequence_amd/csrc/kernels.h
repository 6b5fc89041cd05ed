// Kernel templates of libretention.so (gfx950). Each kernel-group source instantiates a subset and exposes
// getters; the C-ABI source launches them.
#pragma once

#include <type_traits>

#include "retention_device.h"

namespace ret {
// Cache-policy operand of a buffer access with the non-temporal hint (gfx950): for data read or written once,
// which need not stay in the caches.
constexpr int kCachePolicyNT = 2;
}  // namespace ret

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
    void* qr;                // rotated copies of q and k (bf16 single-pass kernel with pre-rotated operands)
    void* kr;
    int B, N, H, dk, dv;
    int nseg;                // segments per sequence
    int seg_len;             // tokens per segment (multiple of the chunk), last segment may be shorter
    long long chain_spin;    // segment-chain wait limit without progress (100 MHz ticks); < 0: give up at once
    int out_bf16;
    int rotate;
    long long pos0;
    // Multi-scale retention epilogue applied to the outputs before they are stored (epi != 0; only kernels
    // that hold whole head rows take it): y = swish(gate) (.) GroupNorm_h(o).
    const void* gate;        // [B,N,H,dv] like o, or null
    const float* gn_weight;  // [H * dv] or null
    const float* gn_bias;    // [H * dv] or null
    float eps;
    int epi, gate_bf16;
    // Output rows turned back by the transpose rotation at their positions (theta, pos0), for kernels that stage
    // q and k as given (the gradients' dq' and dk' retentions); vrot: v rows turned by the rotation at their
    // positions while staged (those retentions' v is K' or Q').
    int orot, vrot;
    // Three-launch bf16 kernels only. qk_din (0: d_k): q and k are columns qk_col0 .. qk_col0 + d_k - 1 of heads
    // qk_din wide, so that a run can take one block of wider heads in place. The full pass alone also takes:
    // qk_blocks > 1: the units run over that many such blocks (block i at columns qk_col0 + i d_k, its outputs
    // o_block elements after block i - 1's); ws_t: each segment enters with the transpose of the state in the
    // slot of its unit and segment there (another run's states, d_k = d_v tile).
    int qk_din, qk_col0, qk_blocks;
    long long o_block;
    const float* ws_t;
    // chunk_fused_bf16 in three launches: 1 = the local passes, 2 = the full passes (0: one chained launch)
    int split;
    float log2g[kMaxHeads];
    double theta[kMaxPairs];
};

// swish(g) = g sigmoid(g), the sigmoid as 1 / (1 + 2^(-g log2 e)) on the hardware 2^x and reciprocal (about
// 1 ulp each).
__device__ __forceinline__ float swish_hw(float g) {
    return g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

// Sum over LPG consecutive lanes (a power of 2, aligned), left in every one of them. Within a row of 16 lanes
// the partner values move by DPP (quad permutations, then the half-row and row mirrors: after the steps
// before, the mirrored lane holds the other half's sum), with no LDS round trip; across rows by shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int LPG>
__device__ __forceinline__ float lanes_sum(float s) {
    if constexpr (LPG >= 2) s += dpp_mov<0xb1>(s);   // quad_perm [1,0,3,2]
    if constexpr (LPG >= 4) s += dpp_mov<0x4e>(s);   // quad_perm [2,3,0,1]
    if constexpr (LPG >= 8) s += dpp_mov<0x141>(s);  // row_half_mirror
    if constexpr (LPG >= 16) s += dpp_mov<0x140>(s); // row_mirror
#pragma unroll
    for (int m = 16; m < LPG; m *= 2) s += __shfl_xor(s, m);
    return s;
}

// GroupNorm of one group of values spread over LPG consecutive lanes (EPL values each, in x): standardized in
// place by the group's mean and biased variance over n values, (x - mean) / sqrt(var + eps).
template <int LPG, int EPL>
__device__ __forceinline__ void group_standardize(float* x, float n, float eps) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) s += x[e];
    s = lanes_sum<LPG>(s);
    const float mean = s / n;
    float s2 = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        x[e] -= mean;
        s2 += x[e] * x[e];
    }
    s2 = lanes_sum<LPG>(s2);
    const float inv = __builtin_amdgcn_rsqf(s2 / n + eps);
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] *= inv;
}

// Workspace of the single-pass chunkwise kernel when a sequence is split into nseg > 1 segments: a header,
// two counters per unit (next segment ticket, workgroups past the look-back), one flag per (unit, segment)
// and two state slots per (unit, segment), the aggregate and the inclusive prefix (slot_floats floats each;
// unit = one d_v tile of one (b, h)). Header, counters and flags must be zero before a run and are zero
// again after it, except the sticky `error` word.
struct ChainHeader {
    int reserved[2];
    int error;  // nonzero: a wait gave up
    int pad[61];
};
struct ChainLayout {
    size_t ctr_off, flags_off, agg_off, inc_off, bytes;
};
// Counters and flags take the first kChainMeta bytes whenever they fit: a call leaves them zero, and the slots of
// any layout start past them, so a workspace can pass between calls of different shapes (units x segments up to
// about 16,000) without being cleared again.
constexpr size_t kChainMeta = 64 * 1024;
__host__ __device__ inline ChainLayout chain_layout(int units, int nseg, int slot_floats) {
    ChainLayout L;
    const size_t nslots = (size_t)units * nseg;
    L.ctr_off = sizeof(ChainHeader);
    L.flags_off = L.ctr_off + ((size_t)units * 8 + 255) / 256 * 256;
    L.agg_off = L.flags_off + (nslots * 4 + 255) / 256 * 256;
    if (L.agg_off < kChainMeta) L.agg_off = kChainMeta;
    L.inc_off = L.agg_off + nslots * slot_floats * 4;
    L.bytes = L.inc_off + nslots * slot_floats * 4;
    return L;
}

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
    // Region A holds sQ, sK and sKc while a chunk's slices are computed. The output tile (fp32 at most) gets
    // its own region when the LDS budget allows (SEP_O): its global stores then overlap the next chunk's
    // staging. Otherwise it reuses region A once the chunk's slices are done.
    static constexpr int A_STAGE = (2 * SQ + SKC) * (int)sizeof(st), A_OUT = C * LDO * 4;
    static constexpr int REST = (SVC + SP + SRT) * (int)sizeof(st);
    static constexpr int WITH_SEP = ((A_STAGE + 15) / 16 * 16) + REST + A_OUT;
    static constexpr int WITHOUT_SEP = ((A_STAGE > A_OUT ? A_STAGE : A_OUT) + 15) / 16 * 16 + REST;
    // (a separate tile must not cost a workgroup per CU: 80 KB is the two-workgroup limit)
    static constexpr bool SEP_O = WITH_SEP <= 160 * 1024 && (WITH_SEP <= 80 * 1024 || WITHOUT_SEP > 80 * 1024);
    static constexpr int A_BYTES = SEP_O ? (A_STAGE + 15) / 16 * 16 : ((A_STAGE > A_OUT ? A_STAGE : A_OUT) + 15) / 16 * 16;
    static constexpr int LDS_BYTES = A_BYTES + REST + (SEP_O ? A_OUT : 0);
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
    char* sO = F::SEP_O ? reinterpret_cast<char*>(sRt + F::SRT) : reinterpret_cast<char*>(smem);  // output tile

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g4 = 4 * (lane >> 4), n16 = lane & 15;
    const int seg = blockIdx.x, dvt = blockIdx.y, pair = blockIdx.z;
    const int b = pair / a.H, h = pair % a.H;
    const int dv0 = dvt * DVT;
    const float lg = a.log2g[h];
    const int osz = a.out_bf16 ? 2 : 4;
    const long long seg_t0 = (long long)seg * a.seg_len;
    const long long seg_t1 = min((long long)a.N, seg_t0 + a.seg_len);
    const int nchunks = (int)((seg_t1 - seg_t0 + C - 1) / C);
    const int nst = nchunks * F::NSL;
    const int rsk = a.H * a.dk, rsv = a.H * a.dv;

    // This thread's staging items: token block and first dim; pointers at the segment's first chunk.
    int qtb[NIQ], qdb[NIQ], vtb[NIV], vdb[NIV];
    const st *qp[NIQ], *kp[NIQ], *vp[NIV];
#pragma unroll
    for (int j = 0; j < NIQ; ++j) {
        const int x = min(tid + kThreads * j, F::IQK::count - 1);
        qtb[j] = x / (F::KS / IQ);
        qdb[j] = x % (F::KS / IQ);
        const long long off = (((long long)b * a.N + seg_t0 + qtb[j] * 8) * a.H + h) * a.dk + qdb[j] * IQ;
        qp[j] = (const st*)a.q + off;
        kp[j] = (const st*)a.k + off;
    }
#pragma unroll
    for (int j = 0; j < NIV; ++j) {
        const int x = min(tid + kThreads * j, F::IV::count - 1);
        vtb[j] = x / (DVT / IVW);
        vdb[j] = x % (DVT / IVW);
        vp[j] = (const st*)a.v + (((long long)b * a.N + seg_t0 + vtb[j] * 8) * a.H + h) * a.dv + dv0 + vdb[j] * IVW;
    }

    // NBUF register buffers: the loads of stage i + NBUF are issued as soon as stage i has been committed.
    // Two buffers where the registers allow it (chunks up to 64 tokens), else one.
    constexpr int NBUF = C <= 64 ? 2 : 1;
    Item<E, IQ> bq[NBUF][NIQ], bk[NBUF][NIQ];
    Item<E, IVW> bv[NBUF][NIV];
    auto issue = [&](int i, auto parc) __attribute__((always_inline)) {
        constexpr int par = decltype(parc)::value;
        const int c = i / F::NSL, sl = i % F::NSL;
        const int L = (int)min((long long)C, seg_t1 - seg_t0 - (long long)c * C);
        const long long cq = (long long)c * C * rsk + sl * F::KS;
#pragma unroll
        for (int j = 0; j < NIQ; ++j)
            if (tid + kThreads * j < F::IQK::count) {
                issue_item<E, IQ>(bq[par][j], qp[j] + cq, rsk, L - qtb[j] * 8);
                issue_item<E, IQ>(bk[par][j], kp[j] + cq, rsk, L - qtb[j] * 8);
            }
        if (sl == 0) {
            const long long cv = (long long)c * C * rsv;
#pragma unroll
            for (int j = 0; j < NIV; ++j)
                if (tid + kThreads * j < F::IV::count) issue_item<E, IVW>(bv[par][j], vp[j] + cv, rsv, L - vtb[j] * 8);
        }
    };
    if (nst > 0) issue(0, std::integral_constant<int, 0>{});
    if constexpr (NBUF == 2)
        if (nst > 1) issue(1, std::integral_constant<int, NBUF - 1>{});

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

    // Scores above the diagonal are never written: keep them zero for the P.V product.
    for (int i = tid; i < F::SP; i += kThreads) sP[i] = (st)0;

    // Decay factors that do not depend on the chunk: the mask gamma^(j-l) of each owned S^T tile (rows l,
    // columns j) and xi_j = gamma^(j+1) of each owned O^T tile (columns j). S^T tiles of this wave: t = w + 4x
    // in row-by-row lower-triangle order.
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
    RotStep<IQ / 2> rstep[NIQ][F::NSL];
    float zfull[NIQ][8];
#pragma unroll
    for (int j = 0; j < NIQ; ++j) {
#pragma unroll
        for (int sl = 0; sl < F::NSL; ++sl)
            if (a.rotate) rstep[j][sl].init(a.theta, (sl * F::KS + qdb[j] * IQ) / 2);
        item_zeta(zfull[j], lg, C - 1 - qtb[j] * 8, 8);
    }
    const float gC = gpow(lg, (float)C);

    // Copy of R (operand precision), transposed to [d_v][d_k], for the cross product.
#pragma unroll
    for (int i = 0; i < F::NR_W; ++i) {
        const int t = w + kWaves * i;
        if (t < F::NR) {
            const int rb = t / F::NDV, cb = t % F::NDV;
            store4(sRt + (cb * 16 + n16) * F::LDR + rb * 16 + g4, R[i]);
        }
    }

    auto commit = [&](int i, auto parc, auto slc) __attribute__((always_inline)) {
        constexpr int par = decltype(parc)::value, sl = decltype(slc)::value;
        const int c = i / F::NSL;
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
                commit_qk<E, IQ, true, true>(&bq[par][j], bk[par][j], L - qtb[j] * 8, a.rotate, a.theta,
                                             (sl * F::KS + qdb[j] * IQ) / 2, a.pos0 + t0 + qtb[j] * 8, rstep[j][sl],
                                             zt, sQ + qtb[j] * 8 * F::LDQ + qdb[j] * IQ, F::LDQ,
                                             sK + qtb[j] * 8 * F::LDQ + qdb[j] * IQ, F::LDQ,
                                             sKc + qdb[j] * IQ * F::LDC + qtb[j] * 8, F::LDC);
            }
        if constexpr (sl == 0) {
#pragma unroll
            for (int j = 0; j < NIV; ++j)
                if (tid + kThreads * j < F::IV::count)
                    commit_vcol<E, IVW>(bv[par][j], L - vtb[j] * 8, sVc + vdb[j] * IVW * F::LDC + vtb[j] * 8, F::LDC);
        }
    };

    // Coalesced 16-byte stores of output rows j < L of the chunk starting at t0 from the output tile.
    auto store_out_tile = [&](long long t0, int L) __attribute__((always_inline)) {
        const int vec = 16 / osz;  // elements per 16-byte store
        const int per_row = DVT / vec;
        char* obase = (char*)a.o + ((((long long)b * a.N + t0) * a.H + h) * a.dv + dv0) * osz;
        for (int x = tid; x < L * per_row; x += kThreads) {
            const int j = x / per_row, c16 = x % per_row;
            *reinterpret_cast<uint4*>(obase + ((long long)j * rsv + c16 * vec) * osz) =
                *reinterpret_cast<const uint4*>(sO + (j * F::LDO + c16 * vec) * osz);
        }
    };
    // With four d_v blocks, each wave's O^T and R tiles share one d_v block, so the operand fragment of that
    // block is read from LDS once per k-step and reused across the wave's tiles.
    constexpr bool SHARED_DV = F::NDV == kWaves;

    // One chunk; cpar is the chunk's parity, so every stage's buffer parity is known at compile time.
    auto chunk = [&](int c, auto cparc) __attribute__((always_inline)) {
        constexpr int cpar = decltype(cparc)::value;
        const long long t0 = seg_t0 + (long long)c * C;
        const int L = (int)min((long long)C, seg_t1 - t0);
        const float gL = L == C ? gC : gpow(lg, (float)L);
        f32x4_t S[F::NS_W], O[F::NO_W];
#pragma unroll
        for (int x = 0; x < F::NS_W; ++x) S[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int x = 0; x < F::NO_W; ++x) O[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        static_for<0, F::NSL>([&](auto slc) __attribute__((always_inline)) {
            constexpr int sl = decltype(slc)::value;
            constexpr int par = NBUF == 2 ? (cpar * F::NSL + sl) & 1 : 0;
            const int i = c * F::NSL + sl;
            // Staging buffers free: for a chunk's first slice with a separate output tile, the barrier that
            // ended the previous chunk already guarantees it.
            if (!(F::SEP_O && sl == 0 && c > 0)) __syncthreads();
            commit(i, std::integral_constant<int, par>{}, slc);
            if (i + NBUF < nst) issue(i + NBUF, std::integral_constant<int, par>{});
            if constexpr (F::SEP_O && sl == 0)
                if (c > 0) store_out_tile(t0 - C, C);  // the previous chunk's output, overlapping this staging
            __syncthreads();
            // S^T += K_s Q_s^T over this wave's lower-triangle tiles (keys l <= queries j). Slots past the last
            // tile repeat it; their results are never stored.
#pragma unroll
            for (int x = 0; x < F::NS_W; ++x)
                mma_nt(S[x], sK + Slb[x] * 16 * F::LDQ, F::LDQ, sQ + Sjb[x] * 16 * F::LDQ, F::LDQ, F::KS, lane);
            // O^T += R_s^T Q_s^T (cross-chunk read of the state carried in from the previous chunk).
            if constexpr (SHARED_DV) {
#pragma unroll
                for (int kk = 0; kk < F::KS; kk += E::KD) {
                    const auto fa = frag(sRt + w * 16 * F::LDR + sl * F::KS, F::LDR, kk, lane);
#pragma unroll
                    for (int x = 0; x < F::NO_W; ++x) mfma(O[x], fa, frag(sQ + x * 16 * F::LDQ, F::LDQ, kk, lane));
                }
            } else {
#pragma unroll
                for (int x = 0; x < F::NO_W; ++x)
                    if (F::NO % kWaves == 0 || w + kWaves * x < F::NO) {
                        const int jb = ojb<F>(w, x), db = odb<F>(w, x);
                        mma_nt(O[x], sRt + db * 16 * F::LDR + sl * F::KS, F::LDR, sQ + jb * 16 * F::LDQ, F::LDQ,
                               F::KS, lane);
                    }
            }
            // R_s <- gamma^L R_s + K_s^T (V (.) zeta): zeta is folded into sKc. R tile x of wave w covers d_k
            // block rb = (w + 4x) / NDV; with four d_v blocks rb = x and the d_v block is the wave's.
            if constexpr (SHARED_DV) {
                constexpr int XB = F::KS / 16;  // this slice's R tiles: x in [sl*XB, (sl+1)*XB)
#pragma unroll
                for (int x = sl * XB; x < (sl + 1) * XB; ++x) R[x] *= gL;
#pragma unroll
                for (int kk = 0; kk < C; kk += E::KD) {
                    const auto fb = frag(sVc + w * 16 * F::LDC, F::LDC, kk, lane);
#pragma unroll
                    for (int x = sl * XB; x < (sl + 1) * XB; ++x)
                        mfma(R[x], frag(sKc + (x - sl * XB) * 16 * F::LDC, F::LDC, kk, lane), fb);
                }
            } else {
#pragma unroll
                for (int x = 0; x < F::NR_W; ++x) {
                    const int t = w + kWaves * x;
                    const int rb = t / F::NDV, cb = t % F::NDV;
                    if ((F::NR % kWaves == 0 || t < F::NR) && rb / (F::KS / 16) == sl) {
                        R[x] *= gL;
                        mma_nt(R[x], sKc + (rb - sl * (F::KS / 16)) * 16 * F::LDC, F::LDC, sVc + cb * 16 * F::LDC,
                               F::LDC, C, lane);
                    }
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
        for (int x = 0; x < F::NO_W; ++x) O[x] *= Xi[x];
        if constexpr (SHARED_DV) {
#pragma unroll
            for (int kk = 0; kk < C; kk += E::KD) {
                const auto fa = frag(sVc + w * 16 * F::LDC, F::LDC, kk, lane);
#pragma unroll
                for (int x = 0; x < F::NO_W; ++x)
                    if (kk < (x + 1) * 16) mfma(O[x], fa, frag(sP + x * 16 * F::LDC, F::LDC, kk, lane));
            }
        }
#pragma unroll
        for (int x = 0; x < F::NO_W; ++x) {
            if (F::NO % kWaves == 0 || w + kWaves * x < F::NO) {
                const int jb = ojb<F>(w, x), db = odb<F>(w, x);
                if constexpr (!SHARED_DV) {
                    const int kmax = min(C, ((jb + 1) * 16 + E::KD - 1) / E::KD * E::KD);
                    mma_nt(O[x], sVc + db * 16 * F::LDC, F::LDC, sP + jb * 16 * F::LDC, F::LDC, kmax, lane);
                }
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
        if constexpr (!F::SEP_O) store_out_tile(t0, L);
    };

    for (int c = 0; c < nchunks; c += 2) {
        chunk(c, std::integral_constant<int, 0>{});
        if (c + 1 < nchunks) chunk(c + 1, std::integral_constant<int, 1>{});
    }
    if constexpr (F::SEP_O)
        if (nchunks > 0) store_out_tile(seg_t0 + (long long)(nchunks - 1) * C, (int)(seg_t1 - seg_t0 - (long long)(nchunks - 1) * C));

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
    auto issue = [&](int i) __attribute__((always_inline)) {
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
    auto commit = [&](int i) __attribute__((always_inline)) {
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
// recurrent_step: one workgroup per (CW-column d_v tile, b*H + h) with one wave per WR state rows (defaults
// CW = 64, WR = 32: two waves per 64-row tile). Lane (rg, cg) of a wave owns columns 4cg..4cg+3 and WR/RG
// consecutive rows (RG = 64 / (CW/4) row groups): it loads q, k, v and the rotation factors of its rows first,
// then its state rows (all in flight at once), rotates q and k, updates each row S = gamma S + k_r v and writes
// it back in place as it goes, while o = q S is summed over its rows, then over the wave's row groups with lane
// shuffles, then over the waves through LDS. The rotation factors cos/sin(pos theta_i) come from the host,
// evaluated there in fp64 once per step.
// ---------------------------------------------------------------------------------------------------
struct StepArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* state;
    int B, H, dk, dv;
    int in_bf16, out_bf16, rotate;
    float gamma[kMaxHeads];
    // cos and sin of pos * theta_i for the step's position, evaluated on the host in fp64
    float rc[kMaxPairs], rs[kMaxPairs];
    // Per-sequence positions (device [B], or null): the factors then come from pos[b] and theta in the kernel.
    const long long* pos;
    double theta[kMaxPairs];
};

__device__ __forceinline__ float ld_in(const void* p, long long i, int bf) {
    return bf ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

// n consecutive input elements (fp32 or bf16) widened to fp32, loaded as 16/8/4-byte vectors.
template <class E, int N>
__device__ __forceinline__ void load_n(const typename E::st* p, float* f) {
    if constexpr (N == 2) {
        if constexpr (sizeof(typename E::st) == 2) {
            const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
            f[0] = __uint_as_float(u << 16);
            f[1] = __uint_as_float(u & 0xffff0000u);
        } else {
            const float2 x = *reinterpret_cast<const float2*>(p);
            f[0] = x.x;
            f[1] = x.y;
        }
    } else if constexpr (sizeof(typename E::st) == 2) {
        static_assert(N % 4 == 0, "bf16 vector loads");
        if constexpr (N % 8 == 0) {
#pragma unroll
            for (int i = 0; i < N; i += 8) load8(p + i, f + i);
        } else {
#pragma unroll
            for (int i = 0; i < N; i += 4) {
                const uint2 u = *reinterpret_cast<const uint2*>(p + i);
                f[i] = __uint_as_float(u.x << 16);
                f[i + 1] = __uint_as_float(u.x & 0xffff0000u);
                f[i + 2] = __uint_as_float(u.y << 16);
                f[i + 3] = __uint_as_float(u.y & 0xffff0000u);
            }
        }
    } else {
        static_assert(N % 4 == 0, "fp32 vector loads");
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const float4 x = *reinterpret_cast<const float4*>(p + i);
            f[i] = x.x;
            f[i + 1] = x.y;
            f[i + 2] = x.z;
            f[i + 3] = x.w;
        }
    }
}

// (b, h) pairs per grouped decode workgroup: as many as fill 8 waves of d_k / wr waves each.
__host__ __device__ constexpr int step_group_pairs(int dk, int wr) { return dk / wr >= 8 ? 1 : 8 / (dk / wr); }

// One decode step for PPW (b, h) pairs and CW state columns: NW waves of WR rows per pair. Lane (rg, cg) of a wave
// owns columns 4cg..4cg+3 of rows rg*RPT .. +RPT-1 (each row segment one 16-byte access, a row's CW columns
// contiguous across the cg lanes). Every address is formed first and every load (q, k, v, the rotation factors,
// then the state rows) issued before any is waited for; each row is updated and written back as soon as it
// arrives, so loads and stores overlap. o sums q_r S_r over the rows (shuffles within a wave, LDS across waves).
// Several pairs share a workgroup of up to 8 waves: fewer, larger workgroups reach the state sooner than many
// small ones. Pairs past B*H (a partial last workgroup) load the last pair and store nothing. NT: the state's
// loads and stores carry the non-temporal hint, for a state that is read and written once per step and not
// again before it has left the caches (one state of many, as one per layer of a model).
template <class E, int DK, int CW, int WR, int PPW, bool POS, bool NT>
__global__ __launch_bounds__(64 * (DK / WR) * PPW) void recurrent_step_kernel(StepArgs a) {
    typedef typename E::st st;
    constexpr int NW = DK / WR;                 // waves per pair
    constexpr int CG = CW / 4;                  // column groups of a wave
    constexpr int RG = 64 / CG;                 // row groups of a wave
    constexpr int RPT = WR / RG;                // rows per lane (pairs of rows stay in one lane)
    static_assert(RPT >= 2 && RPT % 2 == 0 && RG * CG == 64, "decode tile");
    __shared__ float4 part[PPW][NW][CG];
    const int tid = threadIdx.x, lane = tid & 63, wv = (tid >> 6) % NW, sub = tid / (64 * NW);
    const int cg = lane % CG, rg = lane / CG;
    const int npairs = a.B * a.H, dv = a.dv;
    const int pair_id = blockIdx.y * PPW + sub;
    const bool live = pair_id < npairs;
    // wave-uniform: gamma is a scalar read, issued with the kernel arguments
    const int pair = __builtin_amdgcn_readfirstlane(live ? pair_id : npairs - 1);
    const float g = a.gamma[pair % a.H];
    const int c0 = blockIdx.x * CW + 4 * cg;
    const bool active = live && c0 < dv;
    const int cc = c0 < dv ? c0 : 0;    // column of the loads (in range also for idle lanes)
    const int r0 = wv * WR + rg * RPT;  // first row of this lane
    const st* vp = (const st*)a.v + (long long)pair * dv + cc;
    const st* qp = (const st*)a.q + (long long)pair * DK + r0;
    const st* kp = (const st*)a.k + (long long)pair * DK + r0;
    // The pair's state through one buffer resource: row i of the lane at the lane's offset plus a scalar i*dv*4,
    // so the RPT loads go out back to back from one address register. Idle lanes point past the resource:
    // their loads read zeros and their stores are dropped.
    const int sbytes = DK * dv * 4;
    const __amdgpu_buffer_rsrc_t srs =
        __builtin_amdgcn_make_buffer_rsrc(a.state + (long long)pair * DK * dv, (short)0, sbytes, 0x00020000);
    const int svoff = active ? (r0 * dv + c0) * 4 : sbytes;
    float vv[4], qv[RPT], kv[RPT], rc[RPT / 2], rs[RPT / 2];
    // POS: each sequence at its own position pos[b] (a scalar load, issued with the others and used after the
    // state loads); otherwise the call's factors from the kernel arguments
    long long ppos = 0;
    if constexpr (POS) ppos = a.pos[pair / a.H];
    load_n<E, 4>(vp, vv);
    load_n<E, RPT>(qp, qv);
    load_n<E, RPT>(kp, kv);
#pragma unroll
    for (int p = 0; p < RPT / 2; ++p) {  // read also without rotation, so that no branch holds them back
        if constexpr (!POS) {
            rc[p] = a.rc[r0 / 2 + p];
            rs[p] = a.rs[r0 / 2 + p];
        }
    }
    constexpr int cpol = NT ? kCachePolicyNT : 0;
    float4 x[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const f32x4_t t =
            __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(srs, svoff, i * dv * 4, cpol));
        x[i] = make_float4(t[0], t[1], t[2], t[3]);
    }
    // Every row has arrived before the first state store goes out. The compiler's own waits would otherwise let
    // later rows' loads be outstanding behind stores, and count on loads and stores completing in issue order,
    // which holds for loads among themselves only.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any of the work below
    if constexpr (POS) {  // this sequence's own position: factors by rot_cs, as in the chunkwise kernels
#pragma unroll
        for (int p = 0; p < RPT / 2; ++p) rot_cs(ppos, a.theta[r0 / 2 + p], &rc[p], &rs[p]);
    }
    // The pair (r0 + 2p, r0 + 2p + 1) turns by the angle pos * theta_(r0/2 + p); without rotation the inputs
    // pass unchanged (a select, not a branch: the factor loads stay ahead of the state loads).
    const bool rot = a.rotate != 0;
#pragma unroll
    for (int p = 0; p < RPT / 2; ++p) {
        const float c = rc[p], sn = rs[p];
        const float q0 = qv[2 * p], q1 = qv[2 * p + 1], k0 = kv[2 * p], k1 = kv[2 * p + 1];
        qv[2 * p] = rot ? q0 * c - q1 * sn : q0;
        qv[2 * p + 1] = rot ? q0 * sn + q1 * c : q1;
        kv[2 * p] = rot ? k0 * c - k1 * sn : k0;
        kv[2 * p + 1] = rot ? k0 * sn + k1 * c : k1;
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        x[i].x = g * x[i].x + kv[i] * vv[0];
        x[i].y = g * x[i].y + kv[i] * vv[1];
        x[i].z = g * x[i].z + kv[i] * vv[2];
        x[i].w = g * x[i].w + kv[i] * vv[3];
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, f32x4_t{x[i].x, x[i].y, x[i].z, x[i].w}), srs,
                                               svoff, i * dv * 4, cpol);
        acc.x += qv[i] * x[i].x;
        acc.y += qv[i] * x[i].y;
        acc.z += qv[i] * x[i].z;
        acc.w += qv[i] * x[i].w;
    }
    // Sum over the row groups of the wave (lanes CG, 2CG, .. apart).
#pragma unroll
    for (int m = CG; m < 64; m *= 2) {
        acc.x += __shfl_xor(acc.x, m);
        acc.y += __shfl_xor(acc.y, m);
        acc.z += __shfl_xor(acc.z, m);
        acc.w += __shfl_xor(acc.w, m);
    }
    if constexpr (NW > 1) {
        if (rg == 0) part[sub][wv][cg] = acc;
        __syncthreads();
        if (wv != 0) return;
        acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
            const float4 p = part[sub][w2][cg];
            acc.x += p.x;
            acc.y += p.y;
            acc.z += p.z;
            acc.w += p.w;
        }
    }
    if (rg == 0 && active) {
        const long long off = (long long)pair * dv + c0;
        if (a.out_bf16) {
            *reinterpret_cast<uint2*>((uint16_t*)a.o + off) =
                make_uint2(pack2_bf16(acc.x, acc.y), pack2_bf16(acc.z, acc.w));
        } else {
            *reinterpret_cast<float4*>((float*)a.o + off) = acc;
        }
    }
}

}  // namespace ret


namespace ret {

typedef void (*fwd_kernel_t)(FwdArgs);
typedef void (*step_kernel_t)(StepArgs);

// Chunkwise kernels of one shape: either the three-kernel split (local states, segment scan, full pass) or
// one single-pass kernel with the segment chain (fused, non-null).
struct ChunkKernels {
    fwd_kernel_t full, local, fused;
    fwd_kernel_t fused_pre;  // single-pass kernel staging pre-rotated q', k' (or unrotated q, k)
    int dvt;
    // single-pass kernels for chained runs whose segments hold at most seg_tokens tokens (0: none)
    fwd_kernel_t seg, seg_pre;
    fwd_kernel_t seg_rev;  // seg_pre over the reversed sequence (null: none)
    int seg_tokens;
    int threads;      // workgroup size of the fused kernels (0: kThreads)
    int target_wgs;   // workgroups the segment planner aims for (0: the default)
    int threads_pre;  // workgroup size of fused_pre where it differs from `threads` (0: the same)
    int pre_always;   // fused_pre stages operands as given only: with rotation, q and k are rotated up front
                      // whenever the workspace holds the copies
    int pre_only;     // `fused` is fused_pre too: with rotation and no room for rotated copies, the set gives way
                      // to the kernel set of `fallback_variant`
    int fallback_variant;
    const char* pre_name;  // timer name of fused_pre launches (null: the set's default)
    // Three launches instead of one chained one (split_local, split_scan, then fused_pre over every segment),
    // with the segment states in the workspace after its first kChainMeta bytes: split_local, split_scan null
    // otherwise. split_local_rev and split_full_rev run over the reversed sequence (token n of the run is row N-1-n
    // of q, k, v and o; N a multiple of kDmaStep).
    fwd_kernel_t split_local, split_scan, split_local_rev, split_full_rev;
    // fused_pre over the reversed sequence (token n of the run is row N-1-n of q, k, v and o; N a multiple of
    // rev_step), or null
    fwd_kernel_t fused_rev;
    int rev_step;
    // the single-pass kernels run chained segments as three launches instead (FwdArgs::split: the local passes,
    // slot_scan_kernel, the full passes), with the segment states in the workspace after its first kChainMeta bytes
    int fused_split;
    // fused_pre and fused_rev can turn their output rows back by the transpose rotation (FwdArgs::orot) and turn
    // their v rows by the rotation while staging (FwdArgs::vrot)
    int fused_orot;
    // `fused` over the reversed sequence, rotating q and k while staging (null: none), and `seg` likewise
    fwd_kernel_t fused_rot_rev, seg_rot_rev;
};
struct ParKernel {
    fwd_kernel_t fn;
    int bq, dvt;
};

template <class E, int DK, int C, int DVT>
ChunkKernels chunk_entry() {
    ChunkKernels k{};
    k.full = chunk_full_kernel<E, DK, C, DVT>;
    k.local = chunk_local_kernel<E, DK, C, DVT>;
    k.dvt = DVT;
    k.threads = kThreads;
    return k;
}

// Getters, one per kernel-group source. Return false when the shape has no instance.
fwd_kernel_t segment_scan_get();
// W_s = gamma^T W_(s-1) + slot s over a unit's slots (slot 0 holds W_0), in place; grid (slot floats / 512, units)
// of 256 threads.
fwd_kernel_t slot_scan_get();
// q' and k' (bf16): q and k rotated by their absolute positions, into a.qr / a.kr; rotate_qk_blocks() 256-thread
// workgroups.
fwd_kernel_t rotate_qk_get();
constexpr int kRotTokens = 16;  // consecutive tokens per thread of the rotation kernel
inline unsigned rotate_qk_blocks(int B, int N, int H, int dk) {
    const long long threads = (long long)B * ((N + kRotTokens - 1) / kRotTokens) * (H * dk / 8);
    return (unsigned)((threads + 255) / 256);
}
bool chunk_kernels_f32(int dk, int dv, int C, ChunkKernels* out);
bool chunk_kernels_bf16_small(int dk, int dv, int C, ChunkKernels* out);   // d_k in {32, 64}
bool chunk_kernels_bf16_128(int dk, int dv, int C, int variant, ChunkKernels* out);  // d_k = 128
bool chunk_kernels_bf16_256(int dk, int dv, int C, int variant, ChunkKernels* out);  // d_k = 256
// The wide-head kernel (chunk_wide_bf16.h) for d_k in {128, 256} (null otherwise): kWideThreads threads, d_v tiles
// of 128, operands staged as given, steps of kWideStep tokens; rev: over the reversed sequence (N a multiple of
// kWideStep).
constexpr int kWideThreads = 256, kWideStep = 32;
fwd_kernel_t chunk_wide_get(int dk, bool rev = false);
// The LDS-loading wide-head kernels (chunk_dma_bf16.h) for d_k in {128, 256} (false otherwise): the local pass
// (grid units x (segments - 1)) and the full pass (units x segments) of kDmaThreads threads, d_v tiles of kDmaDvt,
// operands staged as given; and the scan between them (grid (d_k * kDmaDvt / 1024, units), 256 threads). The
// local and full passes also over the reversed sequence (local_rev, full_rev).
constexpr int kDmaThreads = 512, kDmaDvt = 256, kDmaStep = 32;  // kDmaStep: tokens per step
struct DmaKernels {
    fwd_kernel_t local, scan, full, local_rev, full_rev;
};
bool chunk_dma_get(int dk, DmaKernels* out);
bool parallel_kernel_get(bool bf16_in, int dk, int dv, ParKernel* out);
// Decode kernel for a (d_k, column tile cw, rows per wave wr) tile, 0 = default, null if none; with pairs_mode 0
// it groups (b, h) pairs into workgroups of up to 8 waves where B*H leaves a workgroup per CU; 1 / 2 force one
// / grouped. The launch is ceil(d_v / cw) x ceil(B*H / ppw) workgroups of 64 * (d_k / wr) * ppw threads.
// positions: the per-sequence-position kernel (default tile only: cw and wr are ignored). stream: the state's
// accesses carry the non-temporal hint, and pairs_mode 0 keeps one pair per workgroup.
step_kernel_t step_kernel_get(bool bf16_in, int dk, int dv, int npairs, int cw, int wr, int pairs_mode,
                              bool positions, bool stream, int* cw_used, int* wr_used, int* ppw_used);

// Multi-scale retention epilogue y = swish(gate) (.) GroupNorm_h(o) over groups of d_v values.
struct EpiArgs {
    const void* o;
    const void* gate;     // null: no gate
    const float* weight;  // [H * dv] or null
    const float* bias;    // [H * dv] or null
    void* y;
    long long groups;  // rows * H
    int H, dv;
    int o_bf16, gate_bf16, y_bf16;
    float eps;
};
typedef void (*epi_kernel_t)(EpiArgs);

// Reordering / rotation of one [B, N, H, d] tensor (d a multiple of 8): output row (b, n, h) is token
// t = out_rev ? N-1-n : n, read from input row in_rev ? N-1-t : t and turned by rot_sign (pos0 + t) theta_i on
// pairs (2i, 2i+1) (rot_sign 0: copied; -1: the transpose rotation). One 256-thread workgroup per 2048 values.
// Reordering and rotation of [B, N, H, d] tensors (the gradients' inputs and outputs). Per token t (rotation
// angle (pos0 + t) theta_i), job j reads row (in_rev ? N-1-t : t) of `in` (columns col0 .. col0 + d - 1 of each
// head of width d_in), adds the same of `in2` if given, and writes row (rev ? N-1-t : t) of out[0] and, if not
// null, of out[1]; rot: +1 turns by the rotation, -1 by its transpose, 0 copies.
struct PermJob {
    const void* in;
    void* out[2];
    int d, rot, in_rev, out_rev[2], in_bf16, out_bf16;
    const void* in2;  // added to `in` before the rotation (same layout and dtype), or null
    int d_in, col0;   // input head width (0: d) and the first input column of each head taken
};
constexpr int kMaxPermJobs = 4;
constexpr int kPermTokens = 4;  // consecutive tokens per thread
struct PermArgs {
    PermJob job[kMaxPermJobs];  // one per blockIdx.y
    int B, N, H;
    long long pos0;
    double theta[kMaxPairs];
};
typedef void (*perm_kernel_t)(PermArgs);
perm_kernel_t permute_rotate_get();
// Zeroes n 32-bit words (a segment chain's counters and flags between calls whose chain layouts differ).
typedef void (*zero_kernel_t)(int*, long long);
zero_kernel_t zero_words_get();
// Kernel for d_v in {16, 32, 64, 128, 256, 512} (null otherwise) and its groups per 256-thread workgroup.
epi_kernel_t epilogue_kernel_get(int dv, int* groups_per_wg);

// Retention score normalizations carried through the decayed key sum z_p = gamma z_{p-1} + k'_p: each output
// row p is the plain row times c_p / den_p, c_p = (1/sqrt(d_k)) (1/sqrt(sum_{i<=p} gamma^i)) for the selected
// factors, den_p = max(|c_p q'_p . z_p|, 1) when the scores are normalized.
struct NormArgs {
    const void* q;       // [B, N, H, dk] (a decode step: [B, H, dk])
    const void* k;
    void* o;             // [B, N, H, dv] (a step: [B, H, dv]), scaled in place
    const float* z_in;   // [B, H, dk] or null (zero)
    float* z_out;        // [B, H, dk] or null
    float* W;            // [B*H][nseg][dk]: local end sums of the segments, then the sums entering them
    float* f;            // [B*N*H] row factors
    int B, N, H, dk, dv;
    int nseg, seg_len;   // the normalization's own segments of the sequence
    int in_bf16, out_bf16, norm, rotate;
    long long pos0;      // absolute position of token 0 (a step: its position)
    float gamma[kMaxHeads];
    double lng[kMaxHeads];           // ln(gamma) in fp64, for the decay row sums
    double theta[kMaxPairs];         // chunkwise: rotation frequencies
    float rc[kMaxPairs], rs[kMaxPairs];  // a step: cos and sin of pos * theta_i from the host
};
constexpr int kNormSegTokens = 256;  // tokens per segment of the chunkwise normalization pass
typedef void (*norm_kernel_t)(NormArgs);
// The normalization kernels for the input dtype and d_k (d_k even, <= 256; null otherwise): the local end sums
// of the segments (one 64-thread workgroup per (segment, b*H + h) for segments 0 .. nseg-2), the row factors (one
// per (segment, b*H + h)), the row scaling (256-thread workgroups over B*N*H*d_v / 8 groups of 8 values), and
// the decode step's factor and key sum update (one 64-thread workgroup per (b, h)).
struct NormKernels {
    norm_kernel_t zseg, rows, scale, step;
};
bool norm_kernels_get(bool bf16_in, int dk, NormKernels* out);

}  // namespace ret
