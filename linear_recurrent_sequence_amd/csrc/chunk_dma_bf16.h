// bf16 chunkwise kernels for wide heads (d_k in {128, 256}) with d_v tiles of 256, on operands staged as given
// (q and k rotated once up front, or no rotation), in three launches instead of one chained launch:
//  1. chunk_dma_local_bf16: every segment but the last runs the state recurrence from zero over its tokens,
//     R_s = sum_t gamma^(L-1-t) k'_t^T v_t (the chunkwise carry without outputs), and stores it in slot s + 1 of
//     its unit (one d_v tile of one (b, h)) in the workspace;
//  2. unit_scan_kernel: per unit and element, slot s becomes the state entering segment s,
//     W_s = gamma^T W_(s-1) + R_(s-1), W_0 = state_in (or 0; T tokens per segment);
//  3. chunk_dma_full_bf16: every segment runs the chunkwise form from W_s (from state_in when the call has one
//     segment), writing the outputs (and the last segment the final state). Only the scan reads state_in when
//     there are several segments, so state_out, written by the last segment, may be the same buffer.
// No workgroup waits for another, so no segment chain is needed, and each kernel holds only what its pass needs.
// The full pass: eight waves, two per SIMD, each owning a d_k x 32 block of the state; 32-token steps; q', k' and v
// rows go from memory straight into the LDS (buffer loads with the LDS bit), three steps deep, waited for with
// explicit counts; the decay weights of the state update, zeta'_l = gamma^-(T + l + 1), are applied to the V^T
// fragments in registers; the state is carried unscaled between rescales (R = gamma^T R^). One d_v tile of 256
// stages the q' and k' rows and computes the causal scores once for 256 columns. The local pass stages k' and v
// through registers (loads straight into the LDS issue too slowly when a step holds only the state update).
// Chunks of 64 or more tokens run as 32-token sub-chunks (the chunkwise form gives the same result for any chunk
// size, up to rounding). For the gradients the kernels also run over the reversed sequence (REV instances), take
// q and k as a block of columns of wider heads (FwdArgs::qk_din, qk_col0), and the full pass runs several such
// blocks in one grid (qk_blocks) and can enter each segment with the transpose of another run's state (ws_t).
#pragma once

#include "chunk_bf16.h"

namespace ret {

template <int DK>
struct DmaB {
    static constexpr int NT = 512, NW = 8;
    static constexpr int C = 32;            // tokens per step
    static constexpr int DVT = 256;         // d_v tile: 8 waves x 32 columns
    static constexpr int NKB = DK / 16;     // d_k blocks of the state
    static constexpr int KS = DK / 32;      // reduction steps over d_k
    static constexpr int NBUF = 3;          // steps of operands resident in the LDS
    typedef Swz<DK> ZQ;
    typedef Swz<DVT> ZV;
    static constexpr int SQ = C * ZQ::LD, SV = C * ZV::LD;  // elements of one q' (k') and one v tile
    static constexpr int BUF = 2 * SQ + SV;                 // one step: sQ, sK, sV
    static constexpr int LDP = C + 8;                       // P rows (query) of 32 keys
    static constexpr int SPB = C * LDP;                     // one P buffer (two: a step's P is read in the next)
    static constexpr int LDS_BYTES = (NBUF * BUF + 2 * SPB) * 2;
    // LDS loads: a tile is C rows of LD / 8 16-byte slots (pads included); one wave instruction fills 64
    // consecutive slots, and instruction i of a tile belongs to wave i % NW.
    static constexpr int NIQ = SQ / 8 / 64, NIV = SV / 8 / 64;
    static constexpr int NIW_Q = (NIQ + NW - 1) / NW, NIW_V = (NIV + NW - 1) / NW;
    // loads per step of wave 0 (the most) and of the last wave (the fewest), with and without the q' tile
    static constexpr int NL_MAX = 2 * NIW_Q + NIW_V, NL_MIN = 2 * (NIQ / NW) + NIV / NW;
    static constexpr int NLK_MIN = NIQ / NW + NIV / NW;
    static constexpr float RESCALE_LOG2 = 64.f;  // largest log2 of gamma^-T before R^ is rescaled
    static_assert(DK == 128 || DK == 256, "wide heads");
    static_assert(SQ % 512 == 0 && SV % 512 == 0, "tiles of whole wave loads");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// s_waitcnt immediates (gfx9 encoding): LDS/scalar counter only, and vector memory counter only.
constexpr int kWaitLgkm0 = 0xC07F;

// Barrier for LDS traffic only: this wave's LDS accesses are complete, and the compiler moves no memory access
// across it. Unlike __syncthreads it does not wait for vector memory (the LDS loads in flight are waited for
// with explicit counts where their data is needed).
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// Raw buffer resource words (stride 0, range-checked dwords: see bytes_rsrc) of a wave-uniform base address.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t rsrc_words(const void* base, int nbytes) {
    const unsigned long long u = reinterpret_cast<unsigned long long>(base);
    return i32x4_t{(int)__builtin_amdgcn_readfirstlane((unsigned)u),
                   (int)(__builtin_amdgcn_readfirstlane((unsigned)(u >> 32)) & 0xffffu),
                   __builtin_amdgcn_readfirstlane(nbytes), kRawBufferWord3};
}
// One 16-byte-per-lane load from a buffer into 64 consecutive LDS slots starting at `lds` (wave-uniform). Written
// as assembly so that the compiler, which cannot tell the LDS buffers apart, does not wait for the load before
// every later LDS read: the kernel waits for these loads itself, with explicit counts. The load has no register
// results; its address registers (and m0, which it reads for the LDS address and which is restored after it)
// are read when it issues.
__device__ __forceinline__ void lds_load16(const i32x4_t& r, uint16_t* lds, int voff) {
    typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
    const unsigned la = __builtin_amdgcn_readfirstlane((unsigned)(unsigned long long)(lds_u16_t*)lds);
    unsigned saved;
    __asm__ volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(la), "v"(voff), "s"(r)
        : "memory");
}

// Byte offset, from a tile's first row in memory, of the global 16-byte segment that LDS slot p of a Swz<W> tile
// holds (row stride `rs` elements; tile row r from memory row r, or from row rows - 1 - r when the tile's `rows`
// rows are taken in reverse); pad slots get an offset past any record count, so they load zeros.
template <int W>
__device__ __forceinline__ int slot_src(int p, int rs, bool flip, int rows) {
    constexpr int SPR = Swz<W>::LD / 8;  // slots per row
    const int r = p / SPR, q = p % SPR;
    if (q >= W / 8) return 0x7ff00000;
    const int s = q ^ ((r >> 3) & 1);   // Swz swaps the two 8-column halves of each 16 in rows 8..15 (mod 16)
    return ((flip ? rows - 1 - r : r) * rs + 8 * s) * 2;
}

// An 8-value bf16 fragment scaled by per-value factors (rounded back to bf16).
__device__ __forceinline__ bf16x8_t scale_frag(bf16x8_t f, const float* z) {
    const u32x4_t u = __builtin_bit_cast(u32x4_t, f);
    float x[8];
    unpack8(u, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= z[e];
    return __builtin_bit_cast(bf16x8_t, pack8(x));
}


// The values every pass of one workgroup shares (REV: the run goes over the reversed sequence).
template <int DK, bool REV>
struct DmaCtx {
    typedef DmaB<DK> F;
    int tid, lane, w, g4, n16;
    int unit, seg, aN, aH, adk, adv, din, anseg, aseg_len, pair, blk, dv0, seg_n, nchunks, rsk, rsv;
    float lg;
    long long seg_t0, hrow;  // hrow: token 0 of this (b, h), in head rows
    __device__ __forceinline__ DmaCtx(const FwdArgs& a) {
        tid = threadIdx.x;
        lane = tid & 63;
        w = wave_id();
        g4 = 4 * (lane >> 4);
        n16 = lane & 15;
        const int ntiles = __builtin_amdgcn_readfirstlane(a.dv / F::DVT);
        const int nblk = __builtin_amdgcn_readfirstlane(a.qk_blocks > 1 ? a.qk_blocks : 1);
        const int units = __builtin_amdgcn_readfirstlane(a.B * a.H * ntiles * nblk);
        unit_seg_of_block(ntiles * nblk, units, &unit, &seg);
        aN = __builtin_amdgcn_readfirstlane(a.N);
        aH = __builtin_amdgcn_readfirstlane(a.H);
        adk = __builtin_amdgcn_readfirstlane(a.dk);
        adv = __builtin_amdgcn_readfirstlane(a.dv);
        anseg = __builtin_amdgcn_readfirstlane(a.nseg);
        aseg_len = __builtin_amdgcn_readfirstlane(a.seg_len);
        pair = unit / (ntiles * nblk);
        blk = unit / ntiles % nblk;
        const int b = pair / aH, h = pair % aH;
        dv0 = (unit % ntiles) * F::DVT;
        lg = a.log2g[h];
        seg_t0 = (long long)seg * aseg_len;
        seg_n = (int)(min((long long)aN, seg_t0 + aseg_len) - seg_t0);
        nchunks = (seg_n + F::C - 1) / F::C;
        din = a.qk_din ? __builtin_amdgcn_readfirstlane(a.qk_din) : adk;
        rsk = aH * din;
        rsv = aH * adv;
        hrow = (long long)b * aN * aH + h;
    }
    // q' or k' (the pre-rotated copies: this unit's block of columns), v and o of this unit's head at its token 0
    // (from there token t is row t)
    __device__ __forceinline__ const uint16_t* qk_head(const void* p, const FwdArgs& a) const {
        return (const uint16_t*)p + hrow * din + __builtin_amdgcn_readfirstlane(a.qk_col0) + blk * adk;
    }
    __device__ __forceinline__ long long v_head() const { return hrow * adv + dv0; }
    __device__ __forceinline__ long long o_head(const FwdArgs& a) const { return blk * a.o_block + v_head(); }
    // The first row in memory of step c's C rows: token seg_t0 + c C of the run, or, over the reversed sequence,
    // row N - seg_t0 - (c + 1) C, whose C rows are then the step's tokens in reverse order.
    __device__ __forceinline__ long long crow(int c) const {
        return REV ? (long long)aN - seg_t0 - (long long)(c + 1) * F::C : seg_t0 + (long long)c * F::C;
    }
    // slot s of this unit (state slots of DK x DVT floats in the thread order of slot_store)
    __device__ __forceinline__ float* slot(const FwdArgs& a, int s) const {
        return a.ws + ((size_t)unit * anseg + s) * (size_t)(DK * F::DVT);
    }
    // R[x * 2 + j][e]: state row x * 16 + g4 + e, column dv0 + (2w + j) * 16 + n16 of the (b, h) state
    __device__ __forceinline__ long long state_index(int x, int j, int e) const {
        return ((long long)pair * DK + x * 16 + g4 + e) * adv + dv0 + (w * 2 + j) * 16 + n16;
    }
};

// R[x * 2 + j][e] = W[(2w + j) 16 + n16][x 16 + g4 + e]: the transpose of a square DK x DK state W that another
// run's slot holds in the thread order of the full pass (slot_store: element (r, c) is component r mod 4 of
// register (r / 16) 2 + (c / 16) mod 2 of thread ((c / 16) / 2) 64 + ((r mod 16) / 4) 16 + c mod 16). For each
// register the four values come from four consecutive threads' vectors, so the 4 loads of a register, issued back
// to back, cover one 1 KB stretch of the slot.
template <int DK>
__device__ __forceinline__ void slot_load_t(const float* src, f32x4_t* R, int w, int g4, int n16) {
    typedef DmaB<DK> F;
    static_assert(DK == F::DVT, "a square state");
    const rsrc_t r = bytes_rsrc(uniform_ptr(src), DK * F::DVT * 4);
    const int lo = ((n16 >> 2) * 16 + g4) * 16 + (n16 & 3) * 4;  // bytes: this lane's thread and component
#pragma unroll
    for (int x = 0; x < F::NKB; ++x)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int xr = (2 * w + j) * 2 + (x & 1);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                R[x * 2 + j][e] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(r, lo, (xr * F::NT + (x >> 1) * 64 + e) * 16, 0));
        }
}

// V^T fragments of wave w's two 16-column blocks of a Swz<256> V tile, scaled by zeta'_r = gamma^-(T + r + 1) for
// the 8 token rows r of the lane's values (4g + i and 16 + 4g + i; zero from row L on).
template <int DVT>
__device__ __forceinline__ void vz_frags(const uint16_t* sV, int L, float T, float lg, int g4, int w, int lv_t,
                                         bf16x8_t* fvz) {
    float z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int r = e < 4 ? g4 + e : 16 + g4 + e - 4;
        z[e] = r < L ? gpow(lg, -(T + (float)(r + 1))) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) fvz[j] = scale_frag(frag_trps<DVT>(sV, 0, (w * 2 + j) * 16, lv_t), z);
}

// ---- 1. the local pass of every segment but the last ----
template <int DK, bool REV>
__global__ __launch_bounds__(512, 1) void chunk_dma_local_bf16(FwdArgs a) {
    typedef DmaB<DK> F;
    constexpr int NT = F::NT, C = F::C, NKB = F::NKB;
    constexpr int NR = NKB * 2;
    typedef typename F::ZQ ZK;
    typedef typename F::ZV ZV;
    typedef RowTile<C, DK, NT> TK;
    typedef RowTile<C, F::DVT, NT> TV;
    constexpr int BUFL = F::SQ + F::SV;  // one step: sK, sV
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BUFL];
    const DmaCtx<DK, REV> x0(a);
    const int tid = x0.tid, lane = x0.lane, w = x0.w, nchunks = x0.nchunks, seg_n = x0.seg_n;
    const int rsk = x0.rsk, rsv = x0.rsv;
    const float lg = x0.lg;
    const uint16_t* kh = x0.qk_head(a.kr, a);
    const uint16_t* vh = (const uint16_t*)a.v + x0.v_head();
    const int lk_t = ZK::lane_trp(lane), lv_t = ZV::lane_trp(lane);
    const int krow = tid / TK::SPR, kseg = tid % TK::SPR, vrow = tid / TV::SPR, vseg = tid % TV::SPR;
    const int koff = (krow * rsk + kseg * 8) * 2, voff = (vrow * rsv + vseg * 8) * 2;
    // the LDS row of the step's memory row r (the rows of a reversed run in reverse order; whole steps only)
    auto lrow = [&](int r) __attribute__((always_inline)) { return REV ? C - 1 - r : r; };

    f32x4_t R[NR];
#pragma unroll
    for (int x = 0; x < NR; ++x) R[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Forward runs take the steps last first: step s adds step n-1-s of the segment (n steps) with the decay of its
    // rows to the segment's end, zeta'_r = gamma^((s+1) C - 1 - r) <= 1 (vz_frags with T = -(s+1) C), so the state
    // needs no rescaling (measured 54 -> 51 us per call on 7b-class-layer). Reversed runs keep the order of the
    // run and carry the state unscaled between rescales, R = gamma^T R^, zeta'_r = gamma^-(T + r + 1): there the
    // other order raised the register count past the limit.
    constexpr bool BACK = !REV;
    float T = BACK ? -(float)C : 0.f;
    auto rescale = [&]() __attribute__((always_inline)) {
        const float f = gpow(lg, T);
#pragma unroll
        for (int x = 0; x < NR; ++x) R[x] *= f;
        T = 0.f;
    };
    // k' and v rows of step st into register set par (LSETS - 1 steps ahead); none past the last step (the
    // resources are empty: the loads read zeros)
    constexpr int LSETS = 3;
    u32x4_t lk[LSETS][TK::NP], lv[LSETS][TV::NP];
    auto lissue = [&](int st, auto parc) __attribute__((always_inline)) {
        constexpr int par = decltype(parc)::value;
        const int c = BACK ? nchunks - 1 - st : st;
        const int L = c >= 0 ? min(C, seg_n - c * C) : 0;
        const long long tc = x0.crow(c >= 0 ? c : 0);
        const rsrc_t rk = bytes_rsrc(kh + tc * rsk, L > 0 ? ((L - 1) * rsk + DK) * 2 : 0);
        const rsrc_t rv = bytes_rsrc(vh + tc * rsv, L > 0 ? ((L - 1) * rsv + F::DVT) * 2 : 0);
#pragma unroll
        for (int p = 0; p < TK::NP; ++p) lk[par][p] = buf_load16(rk, koff, p * TK::RP * rsk * 2);
#pragma unroll
        for (int p = 0; p < TV::NP; ++p) lv[par][p] = buf_load16(rv, voff, p * TV::RP * rsv * 2);
    };
    auto lstep = [&](int st, auto parc) __attribute__((always_inline)) {
        constexpr int par = decltype(parc)::value;
        // a step of C tokens (segments before the last hold whole steps only); in the run's order, rescale first if
        // gamma^-(T + C) could leave the range
        if constexpr (!BACK)
            if (-(T + (float)C) * lg > F::RESCALE_LOG2) rescale();
        // buffer st & 1 was last read by step st - 2, which every wave finished before step st - 1's barrier
        uint16_t* sK = smem + (st & 1) * BUFL;
        uint16_t* sV = sK + F::SQ;
#pragma unroll
        for (int p = 0; p < TK::NP; ++p) lds_store16(sK + ZK::off(lrow(krow + p * TK::RP), kseg * 8), lk[par][p]);
#pragma unroll
        for (int p = 0; p < TV::NP; ++p) lds_store16(sV + ZV::off(lrow(vrow + p * TV::RP), vseg * 8), lv[par][p]);
        lissue(st + LSETS, parc);  // (past the end too: the loads read zeros, and every path counts alike)
        __syncthreads();
        bf16x8_t fvz[2];
        vz_frags<F::DVT>(sV, C, T, lg, x0.g4, w, lv_t, fvz);
        T += BACK ? -(float)C : (float)C;
        // R <- R + K'^T (V (.) zeta') (R^ in the run's order), a ring of 4 K'^T fragments in flight
        constexpr int PD = 4;
        bf16x8_t kr[PD];
#pragma unroll
        for (int x = 0; x < PD; ++x) kr[x] = frag_trps<DK>(sK, 0, x * 16, lk_t);
#pragma unroll
        for (int x = 0; x < NKB; ++x) {
            const bf16x8_t ka = kr[x % PD];
            if (x + PD < NKB) kr[x % PD] = frag_trps<DK>(sK, 0, (x + PD) * 16, lk_t);
#pragma unroll
            for (int j = 0; j < 2; ++j) mfma(R[x * 2 + j], ka, fvz[j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Groups of LSETS steps with no branch inside, so every register set is in the same state on every path
    // around the loop, and the compiler's wait before a step's LDS stores covers that step's loads only; the
    // last steps after it.
    const std::integral_constant<int, 0> set0;
    const std::integral_constant<int, 1> set1;
    const std::integral_constant<int, 2> set2;
    lissue(0, set0);
    lissue(1, set1);
    lissue(2, set2);
    int c = 0;
    for (; c + 2 < nchunks; c += 3) {
        lstep(c, set0);
        lstep(c + 1, set1);
        lstep(c + 2, set2);
    }
    if (c < nchunks) lstep(c, set0);
    if (c + 1 < nchunks) lstep(c + 1, set1);
    if constexpr (!BACK) rescale();
    slot_store<NR, NT>(x0.slot(a, x0.seg + 1), R, tid);
}

// ---- 2. the states entering the segments: W_s = gamma^T W_(s-1) + W_s over s = 1 .. nseg-1 ----
// W_0 = state_in (or 0), gathered into the slots' thread order: the 4 floats at slot offset e are R[xr][0..3] of
// thread t of the full pass (xr = e / (4 NT), t = e / 4 mod NT), state rows x*16 + g4 + 0..3 of column
// dv0 + (2w + j)*16 + n16 (x = xr / 2, j = xr mod 2; w, g4, n16 of t). One thread per 4 consecutive floats of a
// slot, grid (slot floats / 1024, units); the loads of a group of segments are issued together, so the
// dependent chain costs one memory round trip per group.
template <int DK>
__global__ __launch_bounds__(256) void unit_scan_kernel(FwdArgs a) {
    typedef DmaB<DK> F;
    constexpr int G = 8;
    constexpr long long PER = (long long)DK * F::DVT;
    const int unit = blockIdx.y;
    const long long e = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= PER) return;
    const int ntiles = a.dv / F::DVT, nseg = a.nseg;
    const int pair = unit / ntiles, dv0 = (unit % ntiles) * F::DVT;
    const float decay = __builtin_amdgcn_exp2f((float)a.seg_len * a.log2g[pair % a.H]);
    float* W = a.ws + (long long)unit * nseg * PER + e;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.state_in) {
        const int xr = (int)(e / (4 * F::NT)), t = (int)(e / 4 % F::NT);
        const int x = xr / 2, j = xr % 2, w = t / 64, lane = t % 64, g4 = 4 * (lane >> 4), n16 = lane & 15;
        const float* si = a.state_in + ((long long)pair * DK + x * 16 + g4) * a.dv + dv0 + (w * 2 + j) * 16 + n16;
        acc = make_float4(si[0], si[a.dv], si[2 * a.dv], si[3 * a.dv]);
    }
    *reinterpret_cast<float4*>(W) = acc;
    for (int g0 = 1; g0 < nseg; g0 += G) {
        float4 u[G];
#pragma unroll
        for (int j = 0; j < G; ++j)  // past the last segment re-read the last one (unused)
            u[j] = *reinterpret_cast<const float4*>(W + (long long)min(g0 + j, nseg - 1) * PER);
#pragma unroll
        for (int j = 0; j < G; ++j)
            if (g0 + j < nseg) {
                acc.x = decay * acc.x + u[j].x;
                acc.y = decay * acc.y + u[j].y;
                acc.z = decay * acc.z + u[j].z;
                acc.w = decay * acc.w + u[j].w;
                // with no state_in, W_1 = R_0 is slot 1 as the local pass left it
                if (g0 + j > 1 || a.state_in) *reinterpret_cast<float4*>(W + (long long)(g0 + j) * PER) = acc;
            }
    }
}

// ---- 3. the full pass of every segment ----
template <int DK, bool REV>
__global__ __launch_bounds__(512, 1) void chunk_dma_full_bf16(FwdArgs a) {
    typedef DmaB<DK> F;
    constexpr int NT = F::NT, NW = F::NW, C = F::C, NKB = F::NKB, KS = F::KS, NBUF = F::NBUF;
    constexpr int NR = NKB * 2;  // R[x * 2 + j]: d_k block x, d_v block 2w + j of the tile
    typedef typename F::ZQ ZQ;
    typedef typename F::ZV ZV;
    __shared__ __attribute__((aligned(16))) uint16_t smem[F::LDS_BYTES / 2];
    uint16_t* const sP = smem + NBUF * F::BUF;
    const DmaCtx<DK, REV> x0(a);
    const int tid = x0.tid, lane = x0.lane, w = x0.w, g4 = x0.g4, n16 = x0.n16;
    const int seg = x0.seg, nchunks = x0.nchunks, seg_n = x0.seg_n, rsk = x0.rsk, rsv = x0.rsv;
    const float lg = x0.lg;
    const uint16_t* qh = x0.qk_head(a.qr, a);
    const uint16_t* kh = x0.qk_head(a.kr, a);
    const uint16_t* vh = (const uint16_t*)a.v + x0.v_head();
    const int osz = a.out_bf16 ? 2 : 4;
    char* oh = (char*)a.o + x0.o_head(a) * osz;
    const int lq_p = ZQ::lane_p(lane), lq_t = ZQ::lane_trp(lane), lv_t = ZV::lane_trp(lane);

    // The state entering the segment: W_s (the scan of the local passes, state_in included), or state_in itself
    // when the call has one segment; or the transpose of another run's W_s.
    f32x4_t R[NR];
    if (DK == F::DVT && a.ws_t) {  // (square states only)
        if constexpr (DK == F::DVT)
            slot_load_t<DK>(a.ws_t + ((size_t)x0.unit * x0.anseg + seg) * (DK * F::DVT), R, w, g4, n16);
    } else if (x0.anseg > 1) {
        slot_load<NR, NT>(x0.slot(a, seg), R, tid);
    } else {
#pragma unroll
        for (int x = 0; x < NKB; ++x)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    R[x * 2 + j][e] = a.state_in ? a.state_in[x0.state_index(x, j, e)] : 0.f;
    }

    // Every slot starts at zero: rows past a segment's end are loaded as zeros, and no stale or uninitialised
    // value can reach a product even if a load past the end left its slots alone.
    for (int i = tid; i < F::LDS_BYTES / 16; i += NT) lds_store16(smem + 8 * i, u32x4_t{0u, 0u, 0u, 0u});
    __syncthreads();
    // Nothing else in flight from here on but the loads below (the state's loads are consumed above): the
    // explicit counts of wait_step then hold.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

    // this lane's source offsets for the tile slots it fills (instruction i of wave w: slots 64 (w + NW i) + lane)
    int voq[F::NIW_Q], vov[F::NIW_V];
#pragma unroll
    for (int i = 0; i < F::NIW_Q; ++i) voq[i] = slot_src<DK>(64 * (w + NW * i) + lane, rsk, REV, C);
#pragma unroll
    for (int i = 0; i < F::NIW_V; ++i) vov[i] = slot_src<F::DVT>(64 * (w + NW * i) + lane, rsv, REV, C);
    // Loads of step c into LDS buffer c % NBUF; rows past the segment's end read as zero (the resources cover
    // the live rows only; a reversed run has whole steps only). Issued for every step number, past the end too, so the counts below hold. A step's
    // loads go out in three parts (k', q', v rows), so that they can be spread over the products of the step
    // before: issued all at once, the eight waves' loads queue behind each other in the address unit.
    struct Dma {
        i32x4_t rk, rq, rv;
        uint16_t *sQ, *sK, *sV;
    };
    auto dma_of = [&](int c, int buf) __attribute__((always_inline)) {
        Dma d;
        d.sQ = smem + buf * F::BUF;
        d.sK = d.sQ + F::SQ;
        d.sV = d.sK + F::SQ;
        const int L = min(C, seg_n - c * C);
        const long long tc = x0.crow(c);
        d.rk = rsrc_words(kh + tc * rsk, L > 0 ? ((L - 1) * rsk + DK) * 2 : 0);
        d.rq = rsrc_words(qh + tc * rsk, L > 0 ? ((L - 1) * rsk + DK) * 2 : 0);
        d.rv = rsrc_words(vh + tc * rsv, L > 0 ? ((L - 1) * rsv + F::DVT) * 2 : 0);
        return d;
    };
    auto issue_part = [&](const Dma& d, int part) __attribute__((always_inline)) {
        if (part == 0) {
#pragma unroll
            for (int i = 0; i < F::NIW_Q; ++i)
                if (w + NW * i < F::NIQ) lds_load16(d.rk, d.sK + 512 * (w + NW * i), voq[i]);
        } else if (part == 1) {
#pragma unroll
            for (int i = 0; i < F::NIW_Q; ++i)
                if (w + NW * i < F::NIQ) lds_load16(d.rq, d.sQ + 512 * (w + NW * i), voq[i]);
        } else {
#pragma unroll
            for (int i = 0; i < F::NIW_V; ++i)
                if (w + NW * i < F::NIV) lds_load16(d.rv, d.sV + 512 * (w + NW * i), vov[i]);
        }
    };
    auto issue = [&](int c, int buf) __attribute__((always_inline)) {
        const Dma d = dma_of(c, buf);
        issue_part(d, 0);
        issue_part(d, 1);
        issue_part(d, 2);
    };
    // Waits until this wave's loads of the current step have landed, while the next steps' (issued after them)
    // may still be in flight. Vector memory loads complete in order, so with at most the younger steps' loads
    // outstanding none of the current step's is; each wave counts its own loads per step (the first waves hold
    // one instruction more of a tile whose instruction count is not a multiple of the waves).
    auto wait_step = [&]() __attribute__((always_inline)) {
        const int nq = (F::NIQ - w + NW - 1) / NW, nv = (F::NIV - w + NW - 1) / NW;
        const int n = 2 * nq + nv;
        if (n == F::NL_MIN) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(F::NL_MIN * (NBUF - 2)));
        } else if (n == F::NL_MIN + 1) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((F::NL_MIN + 1) * (NBUF - 2)));
        } else if (n == F::NL_MIN + 2) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((F::NL_MIN + 2) * (NBUF - 2)));
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((F::NL_MIN + 3) * (NBUF - 2)));
        }
    };
    static_assert(F::NL_MAX - F::NL_MIN <= 3, "per-wave load counts");
#pragma unroll
    for (int c = 0; c < NBUF - 1; ++c) issue(c, c);

    float T = 0.f;  // tokens of the state since its last rescale (R = gamma^T R^; wave-uniform)
    auto rescale = [&]() __attribute__((always_inline)) {
        const float f = gpow(lg, T);
#pragma unroll
        for (int x = 0; x < NR; ++x) R[x] *= f;
        T = 0.f;
    };
    // decay factors: the mask gamma^(j - l) of this wave's score tile (wave 0: queries 0-15 x keys 0-15, wave
    // 1: queries 16-31 x keys 0-15, wave 2: queries 16-31 x keys 16-31; the other waves have none),
    // xi_j = gamma^(j+1)
    const bool scorer = w < 3;
    const int sjb = w == 0 ? 0 : 1, slb = w == 2 ? 1 : 0;
    f32x4_t DmS;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int jl = 16 * (sjb - slb) + n16 - g4 - e;
        DmS[e] = jl >= 0 ? gpow(lg, (float)jl) : 0.f;
    }
    float Xi[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) Xi[x] = gpow(lg, (float)(x * 16 + n16 + 1));
    // output row x * 16 + n16 of a step: at row x * 16 + n16 of its rows in memory, or reversed at
    // (1 - x) * 16 + 15 - n16
    const int o_voff = ((REV ? 15 - n16 : n16) * rsv + w * 2 * 16 + g4) * osz;
    auto store_out = [&](int c, const f32x4_t* O) __attribute__((always_inline)) {
        const int L = min(C, seg_n - c * C);
        const rsrc_t ro = bytes_rsrc(oh + x0.crow(c) * rsv * osz, ((L - 1) * rsv + F::DVT) * osz);
        if (a.out_bf16) {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    __builtin_amdgcn_raw_buffer_store_b64(
                        __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(2))),
                                           make_uint2(pack2_bf16(O[x * 2 + j][0], O[x * 2 + j][1]),
                                                      pack2_bf16(O[x * 2 + j][2], O[x * 2 + j][3]))),
                        ro, o_voff, ((REV ? 1 - x : x) * 16 * rsv + j * 16) * 2, kOutAux);
        } else {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, O[x * 2 + j]), ro, o_voff,
                                                           ((REV ? 1 - x : x) * 16 * rsv + j * 16) * 4, kOutAux);
        }
    };
    // The P.V product of a step and its output stores run at the start of the next step, after its barrier, which
    // also makes the step's P visible: one barrier per step, and the stores go out ahead of the next loads.
    f32x4_t Op[4];    // the cross term of the previous step, scaled, awaiting its P.V product
    bf16x8_t fvp[2];  // V^T fragments of the previous step (A of P.V)
    auto finish = [&](int c) __attribute__((always_inline)) {
        const uint16_t* sPc = sP + (c & 1) * F::SPB;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int x = 0; x < 2; ++x) mfma(Op[x * 2 + j], fvp[j], frag_p(sPc + x * 16 * F::LDP, F::LDP, 0, lane));
        store_out(c, Op);
    };
    // Step c: wait for its rows, barrier (every wave is past step c - 1: the buffer it used is free, and so is the
    // P buffer of step c - 2), P.V and the output stores of step c - 1, the loads of step c + NBUF - 1 into the
    // free buffer, products, P of the score tiles to LDS.
    int buf = 0;
    for (int c = 0; c < nchunks; ++c) {
        if (-(T + (float)C) * lg > F::RESCALE_LOG2) rescale();
        wait_step();
        lds_barrier();
        if (c > 0) finish(c - 1);
        // step c + NBUF - 1's loads into the buffer step c - 1 used, in three parts during the products below
        const Dma nd = dma_of(c + NBUF - 1, buf == 0 ? NBUF - 1 : buf - 1);
        const uint16_t* sQ = smem + buf * F::BUF;
        const uint16_t* sK = sQ + F::SQ;
        const uint16_t* sV = sK + F::SQ;
        const int L = min(C, seg_n - c * C);
        const float gT = gpow(lg, T);  // scale of the state entering the step
        bf16x8_t fvz[2];
        vz_frags<F::DVT>(sV, L, T, lg, g4, w, lv_t, fvz);
        // One pass over d_k in steps of 32: the cross term O^T = R^T Q'^T (the state entering the step,
        // unscaled), this wave's score tile, and the state update of the two d_k blocks the cross term has just
        // read. Hand-pipelined: step s + 1's fragments are read during step s's products, and a scheduling fence
        // after each step keeps the compiler from hoisting further.
        f32x4_t O[4], S = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int x = 0; x < 4; ++x) O[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        bf16x8_t pq[2][2], pkf[2], pka[2][2];
        auto fetch = [&](int s2, int slot) __attribute__((always_inline)) {
            pq[slot][0] = frag_ps<DK>(sQ, 0, 32 * s2, lq_p);
            pq[slot][1] = frag_ps<DK>(sQ, 16, 32 * s2, lq_p);
            if (scorer) pkf[slot] = frag_ps<DK>(sK, slb * 16, 32 * s2, lq_p);
            pka[slot][0] = frag_trps<DK>(sK, 0, (2 * s2) * 16, lq_t);
            pka[slot][1] = frag_trps<DK>(sK, 0, (2 * s2 + 1) * 16, lq_t);
        };
        fetch(0, 0);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int slot = s & 1;
            if (s + 1 < KS) fetch(s + 1, slot ^ 1);
            if (s * 3 % KS < 3 && s * 3 / KS < 3) issue_part(nd, s * 3 / KS);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bf16x8_t ra = acc_pair(R[(2 * s) * 2 + j], R[(2 * s + 1) * 2 + j]);
                mfma(O[0 * 2 + j], ra, pq[slot][0]);
                mfma(O[1 * 2 + j], ra, pq[slot][1]);
            }
            if (scorer) mfma(S, pkf[slot], sjb == 0 ? pq[slot][0] : pq[slot][1]);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                mfma(R[(2 * s) * 2 + j], pka[slot][0], fvz[j]);
                mfma(R[(2 * s + 1) * 2 + j], pka[slot][1], fvz[j]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        T += (float)L;
        if (scorer) store4(sP + (c & 1) * F::SPB + (sjb * 16 + n16) * F::LDP + slb * 16 + g4, S * DmS);
        // O^T = gamma^T xi (.) O^T + V^T P^T: the first term now, the second at the next step's start (the V rows
        // are read now: the buffer takes new loads in the next step)
#pragma unroll
        for (int x = 0; x < 4; ++x) Op[x] = O[x] * (gT * Xi[x / 2]);
#pragma unroll
        for (int j = 0; j < 2; ++j) fvp[j] = frag_trps<F::DVT>(sV, 0, (w * 2 + j) * 16, lv_t);
        buf = buf == NBUF - 1 ? 0 : buf + 1;
    }
    if (nchunks > 0) {
        lds_barrier();
        finish(nchunks - 1);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the loads past the end have landed before the waves end

    if (seg == x0.anseg - 1 && a.state_out) {
        rescale();
#pragma unroll
        for (int x = 0; x < NKB; ++x)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) a.state_out[x0.state_index(x, j, e)] = R[x * 2 + j][e];
    }
}

}  // namespace ret
