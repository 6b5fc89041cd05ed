// bf16 chunkwise kernel for wide heads (d_k in {128, 256}) with d_v tiles of 256, on operands staged as given
// (q and k rotated once up front, or no rotation). Same computation, state bookkeeping and segment chain as the
// four-wave wide kernel (chunk_wide_bf16.h); what differs is how operands reach the LDS and how many waves share
// them:
//  * eight waves, two per SIMD, each owning a d_k x 32 block of the state; one workgroup per compute unit, so
//    every SIMD has a second wave to issue while one waits on the LDS;
//  * q', k' and v rows go from memory straight into the LDS (buffer loads with the LDS bit: no staging
//    registers, no copy instructions), three steps deep: the loads of step c + 2 are issued when step c starts
//    and waited for with explicit counts, so a step's operands have two steps' time to arrive;
//  * the decay weights of the state update, zeta'_l = gamma^-(T + l + 1), are applied to the V^T fragments in
//    registers (16 values per lane and step) instead of to a scaled copy of V in the LDS;
//  * one d_v tile of 256 stages the q' and k' rows and computes the causal scores once for 256 columns.
// Chunks of 64 or more tokens run as 32-token sub-chunks.
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
    static constexpr int LDS_BYTES = (NBUF * BUF + C * LDP) * 2;
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

// Byte offset, from a tile's first row, of the global 16-byte segment that LDS slot p of a Swz<W> tile holds
// (row stride `rs` elements); pad slots get an offset past any record count, so they load zeros.
template <int W>
__device__ __forceinline__ int slot_src(int p, int rs) {
    constexpr int SPR = Swz<W>::LD / 8;  // slots per row
    const int r = p / SPR, q = p % SPR;
    if (q >= W / 8) return 0x7ff00000;
    const int s = q ^ ((r >> 3) & 1);   // Swz swaps the two 8-column halves of each 16 in rows 8..15 (mod 16)
    return (r * rs + 8 * s) * 2;
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

template <int DK>
__global__ __launch_bounds__(512, 1) void chunk_dma_bf16(FwdArgs a) {
    typedef DmaB<DK> F;
    constexpr int NT = F::NT, NW = F::NW, C = F::C, NKB = F::NKB, KS = F::KS, NBUF = F::NBUF;
    constexpr int NR = NKB * 2;  // R[x * 2 + j]: d_k block x, d_v block 2w + j of the tile
    typedef typename F::ZQ ZQ;
    typedef typename F::ZV ZV;
    __shared__ __attribute__((aligned(16))) uint16_t smem[F::LDS_BYTES / 2];
    __shared__ int s_word;  // broadcast word (ticket, counts)
    uint16_t* const sP = smem + NBUF * F::BUF;

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g4 = 4 * (lane >> 4), n16 = lane & 15;
    const int ntiles = __builtin_amdgcn_readfirstlane(a.dv / F::DVT);
    const int units = __builtin_amdgcn_readfirstlane(a.B * a.H * ntiles);
    const bool chained = a.nseg > 1;
    const int unit = unit_of_block(ntiles, units);
    int seg = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / (unsigned)units));
    Chain ch{};
    if (chained) {
        ch = chain_of(a.ws, units, a.nseg, unit, DK * F::DVT, a.chain_spin);
        seg = chain_ticket(ch, s_word);
    }
    const int aN = __builtin_amdgcn_readfirstlane(a.N);
    const int aH = __builtin_amdgcn_readfirstlane(a.H), adk = __builtin_amdgcn_readfirstlane(a.dk);
    const int adv = __builtin_amdgcn_readfirstlane(a.dv), anseg = __builtin_amdgcn_readfirstlane(a.nseg);
    const int aseg_len = __builtin_amdgcn_readfirstlane(a.seg_len);
    const int pair = unit / ntiles;
    const int b = pair / aH, h = pair % aH;
    const int dv0 = (unit % ntiles) * F::DVT;
    const float lg = a.log2g[h];
    const long long seg_t0 = (long long)seg * aseg_len;
    const int seg_n = (int)(min((long long)aN, seg_t0 + aseg_len) - seg_t0);
    const int nchunks = (seg_n + C - 1) / C;
    const int rsk = aH * adk, rsv = aH * adv;
    const long long head0 = ((long long)b * aN + seg_t0) * aH + h;
    const uint16_t* qh = (const uint16_t*)a.qr + head0 * adk;
    const uint16_t* kh = (const uint16_t*)a.kr + head0 * adk;
    const uint16_t* vh = (const uint16_t*)a.v + head0 * adv + dv0;
    const int osz = a.out_bf16 ? 2 : 4;
    char* oh = (char*)a.o + (head0 * adv + dv0) * osz;
    const int lq_p = ZQ::lane_p(lane), lq_t = ZQ::lane_trp(lane), lv_t = ZV::lane_trp(lane);

    // Every slot starts at zero: rows past a segment's end are loaded as zeros, and no stale or uninitialised
    // value can reach a product even if a load past the end left its slots alone.
    for (int i = tid; i < F::LDS_BYTES / 16; i += NT) lds_store16(smem + 8 * i, u32x4_t{0u, 0u, 0u, 0u});
    __syncthreads();

    // this lane's source offsets for the tile slots it fills (instruction i of wave w: slots 64 (w + NW i) + lane)
    int voq[F::NIW_Q], vov[F::NIW_V];
#pragma unroll
    for (int i = 0; i < F::NIW_Q; ++i) voq[i] = slot_src<DK>(64 * (w + NW * i) + lane, rsk);
#pragma unroll
    for (int i = 0; i < F::NIW_V; ++i) vov[i] = slot_src<F::DVT>(64 * (w + NW * i) + lane, rsv);
    // Loads of step c into LDS buffer c % NBUF; rows past the segment's end read as zero (the resources cover
    // the live rows only). Issued for every step number, past the end too, so the counts below hold.
    auto issue = [&](int c, int buf, auto withq) __attribute__((always_inline)) {
        uint16_t* sQ = smem + buf * F::BUF;
        uint16_t* sK = sQ + F::SQ;
        uint16_t* sV = sK + F::SQ;
        const int L = min(C, seg_n - c * C);
        const long long tc = (long long)c * C;
        const i32x4_t rk = rsrc_words(kh + tc * rsk, L > 0 ? ((L - 1) * rsk + DK) * 2 : 0);
        const i32x4_t rv = rsrc_words(vh + tc * rsv, L > 0 ? ((L - 1) * rsv + F::DVT) * 2 : 0);
#pragma unroll
        for (int i = 0; i < F::NIW_Q; ++i)
            if (w + NW * i < F::NIQ) lds_load16(rk, sK + 512 * (w + NW * i), voq[i]);
        if constexpr (decltype(withq)::value) {
            const i32x4_t rq = rsrc_words(qh + tc * rsk, L > 0 ? ((L - 1) * rsk + DK) * 2 : 0);
#pragma unroll
            for (int i = 0; i < F::NIW_Q; ++i)
                if (w + NW * i < F::NIQ) lds_load16(rq, sQ + 512 * (w + NW * i), voq[i]);
        }
#pragma unroll
        for (int i = 0; i < F::NIW_V; ++i)
            if (w + NW * i < F::NIV) lds_load16(rv, sV + 512 * (w + NW * i), vov[i]);
    };
    // Waits until this wave's loads of the current step have landed, while the next step's (issued after them)
    // may still be in flight. Vector memory loads complete in order, so with at most `n` younger loads
    // outstanding none of the current step's is; each wave counts its own loads per step (the first waves hold
    // one instruction more of a tile whose instruction count is not a multiple of the waves).
    auto wait_step = [&](auto withq) __attribute__((always_inline)) {
        constexpr bool Q = decltype(withq)::value;
        constexpr int NMIN = Q ? F::NL_MIN : F::NLK_MIN;
        const int nq = (F::NIQ - w + NW - 1) / NW, nv = (F::NIV - w + NW - 1) / NW;
        const int n = (Q ? 2 * nq : nq) + nv;
        if (n == NMIN) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(NMIN * (NBUF - 2)));
        } else if (n == NMIN + 1) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((NMIN + 1) * (NBUF - 2)));
        } else if (n == NMIN + 2) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((NMIN + 2) * (NBUF - 2)));
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((NMIN + 3) * (NBUF - 2)));
        }
    };
    static_assert(F::NL_MAX - F::NL_MIN <= 3, "per-wave load counts");

    auto load_state_in = [&](f32x4_t* R) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < NKB; ++x)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    R[x * 2 + j][e] = a.state_in[((long long)pair * DK + x * 16 + g4 + e) * adv + dv0 +
                                                 (w * 2 + j) * 16 + n16];
    };
    f32x4_t R[NR];
#pragma unroll
    for (int x = 0; x < NR; ++x) R[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (seg == 0 && a.state_in) load_state_in(R);
    const bool last = seg == anseg - 1;
    const bool boundary = seg % kChainGroup == kChainGroup - 1;

    // Tokens of the state since its last rescale (R = gamma^T R^; wave-uniform).
    float T = 0.f;
    auto rescale = [&]() __attribute__((always_inline)) {
        const float f = gpow(lg, T);
#pragma unroll
        for (int x = 0; x < NR; ++x) R[x] *= f;
        T = 0.f;
    };
    auto need_rescale = [&](int L) __attribute__((always_inline)) { return -(T + (float)L) * lg > F::RESCALE_LOG2; };
    // zeta' of the 8 tokens of this lane's V^T fragment values (rows 4g + i and 16 + 4g + i), up to gamma^-T
    float zb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) zb[e] = gpow(lg, -(float)((e < 4 ? g4 + e : 16 + g4 + e - 4) + 1));
    // V^T fragments of this wave's two 16-column blocks, scaled by zeta' (zero past the step's last row)
    auto vz_frags = [&](const uint16_t* sV, int L, bf16x8_t* fvz) __attribute__((always_inline)) {
        const float fT = gpow(lg, -T);
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (e < 4 ? g4 + e : 16 + g4 + e - 4) < L ? zb[e] * fT : 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) fvz[j] = scale_frag(frag_trps<F::DVT>(sV, 0, (w * 2 + j) * 16, lv_t), z);
    };
    // R^ <- R^ + K'^T (V (.) zeta') from LDS buffer buf (local pass), a ring of 4 K'^T fragments in flight.
    auto state_update = [&](const uint16_t* sK, const bf16x8_t* fvz) __attribute__((always_inline)) {
        constexpr int PD = 4;
        bf16x8_t kr[PD];
#pragma unroll
        for (int x = 0; x < PD; ++x) kr[x] = frag_trps<DK>(sK, 0, x * 16, lq_t);
#pragma unroll
        for (int x = 0; x < NKB; ++x) {
            const bf16x8_t ka = kr[x % PD];
            if (x + PD < NKB) kr[x % PD] = frag_trps<DK>(sK, 0, (x + PD) * 16, lq_t);
#pragma unroll
            for (int j = 0; j < 2; ++j) mfma(R[x * 2 + j], ka, fvz[j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- local pass over the segment (chained runs, all segments but the last): the state only ----
    if (chained && !last) {
        const std::integral_constant<bool, false> noq;
#pragma unroll
        for (int c = 0; c < NBUF - 1; ++c) issue(c, c, noq);
        int buf = 0;
        for (int c = 0; c < nchunks; ++c) {
            if (need_rescale(C)) rescale();  // (segments before the last hold whole steps only)
            wait_step(noq);
            lds_barrier();  // step c's rows are in; every wave is past step c - 1
            issue(c + NBUF - 1, buf == 0 ? NBUF - 1 : buf - 1, noq);  // into the buffer step c - 1 used
            const uint16_t* sK = smem + buf * F::BUF + F::SQ;
            bf16x8_t fvz[2];
            vz_frags(sK + F::SQ, C, fvz);
            state_update(sK, fvz);
            T += (float)C;
            buf = buf == NBUF - 1 ? 0 : buf + 1;
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the loads past the end have landed too
        lds_barrier();
        rescale();  // the true end state
        // publish the aggregate; the first segment reloads state_in before its flag rises (state_out may be the
        // same buffer, and the last segment writes it only after every earlier flag)
        if (!boundary) {
            if (seg == 0 && a.state_in)
                chain_publish<NR, NT, 0>(ch, seg, R, [&] { load_state_in(R); });
            else
                chain_publish<NR, NT>(ch, seg, R);
        }
    }

    // ---- full pass ----
    const std::integral_constant<bool, true> withq;
#pragma unroll
    for (int c = 0; c < NBUF - 1; ++c) issue(c, c, withq);
    if (chained) {
        f32x4_t Rin[NR];
        chain_enter<NR, NT, true>(ch, seg, anseg, gpow(lg, (float)aseg_len), R, Rin, s_word);
        if (seg > 0 || !a.state_in) {
#pragma unroll
            for (int x = 0; x < NR; ++x) R[x] = Rin[x];
        }
    }
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
    const int o_voff = (n16 * rsv + w * 2 * 16 + g4) * osz;
    auto store_out = [&](int c, const f32x4_t* O) __attribute__((always_inline)) {
        const int L = min(C, seg_n - c * C);
        const rsrc_t ro = bytes_rsrc(oh + (long long)c * C * rsv * osz, ((L - 1) * rsv + F::DVT) * osz);
        if (a.out_bf16) {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    __builtin_amdgcn_raw_buffer_store_b64(
                        __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(2))),
                                           make_uint2(pack2_bf16(O[x * 2 + j][0], O[x * 2 + j][1]),
                                                      pack2_bf16(O[x * 2 + j][2], O[x * 2 + j][3]))),
                        ro, o_voff, (x * 16 * rsv + j * 16) * 2, kOutAux);
        } else {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, O[x * 2 + j]), ro, o_voff,
                                                           (x * 16 * rsv + j * 16) * 4, kOutAux);
        }
    };
    // Step c: wait for its rows, barrier (every wave is past step c - 1, so the buffer it used and sP are free),
    // the loads of step c + NBUF - 1 into that buffer, products, P of the score tiles to LDS, barrier, P.V and the
    // output stores.
    int buf = 0;
    for (int c = 0; c < nchunks; ++c) {
        if (need_rescale(C)) rescale();
        wait_step(withq);
        lds_barrier();
        issue(c + NBUF - 1, buf == 0 ? NBUF - 1 : buf - 1, withq);
        const uint16_t* sQ = smem + buf * F::BUF;
        const uint16_t* sK = sQ + F::SQ;
        const uint16_t* sV = sK + F::SQ;
        const int L = min(C, seg_n - c * C);
        const float gT = gpow(lg, T);  // scale of the state entering the step
        bf16x8_t fvz[2];
        vz_frags(sV, L, fvz);
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
        if (scorer) store4(sP + (sjb * 16 + n16) * F::LDP + slb * 16 + g4, S * DmS);
        lds_barrier();
        // O^T = gamma^T xi (.) O^T + V^T P^T
#pragma unroll
        for (int x = 0; x < 4; ++x) O[x] *= gT * Xi[x / 2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const bf16x8_t fv = frag_trps<F::DVT>(sV, 0, (w * 2 + j) * 16, lv_t);
#pragma unroll
            for (int x = 0; x < 2; ++x) mfma(O[x * 2 + j], fv, frag_p(sP + x * 16 * F::LDP, F::LDP, 0, lane));
        }
        store_out(c, O);
        buf = buf == NBUF - 1 ? 0 : buf + 1;
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the loads past the end have landed before the waves end

    if (last && a.state_out) {
        rescale();
        float* out = a.state_out + (long long)pair * DK * adv;
#pragma unroll
        for (int x = 0; x < NKB; ++x)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    out[(long long)(x * 16 + g4 + e) * adv + dv0 + (w * 2 + j) * 16 + n16] = R[x * 2 + j][e];
    }
}

}  // namespace ret
