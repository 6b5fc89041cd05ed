// bf16 chunkwise kernel for wide heads (d_k in {128, 256}, d_v tiles of 128) on operands staged as given
// (q and k rotated once up front, or no rotation). Same computation and segment chain as chunk_fused_bf16
// (chunk_bf16.h); what differs is how the products meet the LDS:
//  * four waves, one per SIMD, each owning a d_k x 32 block of the state (two 16-column blocks): every Q' row
//    fragment read for the cross term feeds two MFMAs, and so does every K'^T fragment of the state update;
//  * 32-token chunk steps with the whole d_k of Q' and K' staged, double-buffered: two barriers per step;
//  * the Q' fragments of the cross term are also the query operands of the three causal score tiles of a step,
//    which three waves compute (one tile each, over the whole d_k) and hand over as P through LDS;
//  * the state is carried unscaled between rescales: R = gamma^T R^, T the tokens since the last rescale, so a
//    step adds K'^T (V (.) zeta') to R^ with zeta'_l = gamma^-(T + l + 1) and never multiplies R itself (a vector
//    pass over 128 registers per step otherwise); the cross term takes gamma^T with xi. R^ is rescaled (R^ <-
//    gamma^T R^, T = 0) before gamma^-T could exceed 2^64, and before it is published or stored.
// Chunks of 64 or more tokens run as 32-token sub-chunks (the chunkwise form gives the same result for any chunk
// size, up to rounding). REV runs the recurrence over the reversed sequence in place (token n of the run is row
// N-1-n of q, k, v and o; whole steps only, N a multiple of 32): the gradients' retentions over later tokens.
#pragma once

#include "chunk_bf16.h"

namespace ret {

template <int DK>
struct WideB {
    static constexpr int NT = 256, NW = 4;
    static constexpr int C = 32;            // tokens per step
    static constexpr int DVT = 128;         // d_v tile: 4 waves x 32 columns
    static constexpr int NDW = 2;           // 16-column blocks per wave
    static constexpr int NKB = DK / 16;     // d_k blocks of the state
    static constexpr int KS = DK / 32;      // reduction steps over d_k
    typedef RowTile<C, DK, NT> TQ;          // q' and k' rows of a step
    typedef RowTile<C, DVT, NT> TV;         // v rows of the d_v tile
    typedef Swz<DK> ZQ;
    typedef Swz<DVT> ZV;
    static constexpr int SQ = C * ZQ::LD, SV = C * ZV::LD;
    static constexpr int LDP = C + 8;       // P rows (query) of 32 keys
    static constexpr int BUF = 2 * SQ + 2 * SV;  // one step's sQ, sK, sV, sVz (elements)
    static constexpr int LDS_BYTES = (2 * BUF + C * LDP) * 2;
    static constexpr float RESCALE_LOG2 = 64.f;  // largest log2 of gamma^-T before R^ is rescaled
    static_assert(DK == 128 || DK == 256, "wide heads");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int DK, bool REV>
__global__ __launch_bounds__(256, (DK <= 128 ? 2 : 1)) void chunk_wide_bf16(FwdArgs a) {
    typedef WideB<DK> F;
    constexpr int NT = F::NT, C = F::C, NKB = F::NKB, KS = F::KS;
    constexpr int NR = NKB * 2;  // R[x * 2 + j]: d_k block x, d_v block 2w + j of the tile
    typedef typename F::TQ TQ;
    typedef typename F::TV TV;
    typedef typename F::ZQ ZQ;
    typedef typename F::ZV ZV;
    __shared__ __attribute__((aligned(16))) uint16_t smem[F::LDS_BYTES / 2];
    __shared__ int s_word;  // broadcast word (ticket, counts)
    uint16_t* const sP = smem + 2 * F::BUF;

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
    // token 0 of this (b, h), in head rows; the first row in memory of step c: token seg_t0 + c C of the run, or,
    // over the reversed sequence, row N - seg_t0 - (c + 1) C, whose C rows are the step's tokens in reverse order
    const long long hrow = (long long)b * aN * aH + h;
    auto crow = [&](int c) __attribute__((always_inline)) {
        return REV ? (long long)aN - seg_t0 - (long long)(c + 1) * C : seg_t0 + (long long)c * C;
    };
    const uint16_t* qh = (const uint16_t*)a.qr + hrow * adk;
    const uint16_t* kh = (const uint16_t*)a.kr + hrow * adk;
    const uint16_t* vh = (const uint16_t*)a.v + hrow * adv + dv0;
    const int osz = a.out_bf16 ? 2 : 4;
    char* oh = (char*)a.o + (hrow * adv + dv0) * osz;
    // the step's row (and LDS row) of memory row r of its rows
    auto lrow = [&](int r) __attribute__((always_inline)) { return REV ? C - 1 - r : r; };

    // staging: thread t moves 16-byte row segments: q'/k' rows qrow + 8p (segment qseg), v rows vrow + 16p
    const int qrow = tid / TQ::SPR, qseg = tid % TQ::SPR;
    const int qoff = (qrow * rsk + qseg * 8) * 2;
    const int vrow = tid / TV::SPR, vseg = tid % TV::SPR;
    const int voff = (vrow * rsv + vseg * 8) * 2;
    const int lq_p = ZQ::lane_p(lane), lq_t = ZQ::lane_trp(lane), lv_t = ZV::lane_trp(lane);

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

    // Loads of step c into register set par: rows past the segment's end read as zero (the resources cover
    // the live rows only).
    u32x4_t bq[2][TQ::NP], bk[2][TQ::NP], bv[2][TV::NP];
    auto issue = [&](int c, auto parc, auto withq) __attribute__((always_inline)) {
        constexpr int par = decltype(parc)::value;
        const int L = min(C, seg_n - c * C);
        const long long tc = crow(c);
        const rsrc_t rk = bytes_rsrc(kh + tc * rsk, L > 0 ? ((L - 1) * rsk + DK) * 2 : 0);
        const rsrc_t rv = bytes_rsrc(vh + tc * rsv, L > 0 ? ((L - 1) * rsv + F::DVT) * 2 : 0);
#pragma unroll
        for (int p = 0; p < TQ::NP; ++p) bk[par][p] = buf_load16(rk, qoff, p * TQ::RP * rsk * 2);
        if constexpr (decltype(withq)::value) {
            const rsrc_t rq = bytes_rsrc(qh + tc * rsk, L > 0 ? ((L - 1) * rsk + DK) * 2 : 0);
#pragma unroll
            for (int p = 0; p < TQ::NP; ++p) bq[par][p] = buf_load16(rq, qoff, p * TQ::RP * rsk * 2);
        }
#pragma unroll
        for (int p = 0; p < TV::NP; ++p) bv[par][p] = buf_load16(rv, voff, p * TV::RP * rsv * 2);
    };
    // Tokens of the state since its last rescale (R = gamma^T R^; wave-uniform).
    float T = 0.f;
    auto rescale = [&]() __attribute__((always_inline)) {
        const float f = gpow(lg, T);
#pragma unroll
        for (int x = 0; x < NR; ++x) R[x] *= f;
        T = 0.f;
    };
    // Step c's registers into LDS buffer c & 1: q' and k' rows, v rows, and v scaled by zeta'_r = gamma^-(T+r+1)
    // (the state's scale; zero past the step's last row).
    auto commit = [&](int c, auto parc, auto withq) __attribute__((always_inline)) {
        constexpr int par = decltype(parc)::value;
        uint16_t* sQ = smem + (c & 1) * F::BUF;
        uint16_t* sK = sQ + F::SQ;
        uint16_t* sV = sK + F::SQ;
        uint16_t* sVz = sV + F::SV;
        const int L = min(C, seg_n - c * C);
#pragma unroll
        for (int p = 0; p < TQ::NP; ++p) {
            lds_store16(sK + ZQ::off(lrow(qrow + p * TQ::RP), qseg * 8), bk[par][p]);
            if constexpr (decltype(withq)::value)
                lds_store16(sQ + ZQ::off(lrow(qrow + p * TQ::RP), qseg * 8), bq[par][p]);
        }
#pragma unroll
        for (int p = 0; p < TV::NP; ++p) {
            const int r = lrow(vrow + p * TV::RP);
            lds_store16(sV + ZV::off(r, vseg * 8), bv[par][p]);
            const float z = r < L ? gpow(lg, -(T + (float)(r + 1))) : 0.f;
            float vf[8];
            unpack8(bv[par][p], vf);
#pragma unroll
            for (int e = 0; e < 8; ++e) vf[e] *= z;
            lds_store16(sVz + ZV::off(r, vseg * 8), pack8(vf));
        }
    };
    // R^ <- R^ + K'^T (V (.) zeta') from LDS buffer buf. Software-pipelined by hand: the K'^T fragment of block
    // x + 1 is read while block x's products run, and a scheduling fence after each block keeps the compiler from
    // hoisting every read to the top (which would hold all fragments in registers at once).
    // (local pass: a ring of PD fragments in flight, since a block has only two products to cover a read)
    auto state_update = [&](int buf) __attribute__((always_inline)) {
        constexpr int PD = 4;
        const uint16_t* sK = smem + buf * F::BUF + F::SQ;
        const uint16_t* sVz = sK + F::SQ + F::SV;
        bf16x8_t fvz[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) fvz[j] = frag_trps<F::DVT>(sVz, 0, (w * 2 + j) * 16, lv_t);
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
    // a step of L tokens: rescale first if gamma^-(T + L) could leave the range, then T grows by L
    auto need_rescale = [&](int L) __attribute__((always_inline)) { return -(T + (float)L) * lg > F::RESCALE_LOG2; };

    // ---- local pass over the segment (chained runs, all segments but the last): the state only ----
    if (chained && !last) {
        const std::integral_constant<bool, false> noq;
        issue(0, std::integral_constant<int, 0>{}, noq);
        if (nchunks > 1) issue(1, std::integral_constant<int, 1>{}, noq);
        // Buffer c & 1 was last read by step c - 2, which every wave finished before step c - 1's barrier.
        auto lstep = [&](int c, auto parc) __attribute__((always_inline)) {
            if (need_rescale(C)) rescale();  // (segments before the last hold whole steps only)
            commit(c, parc, noq);
            if (c + 2 < nchunks) issue(c + 2, parc, noq);
            __syncthreads();
            state_update(c & 1);
            T += (float)C;
        };
        for (int c = 0; c < nchunks; c += 2) {
            lstep(c, std::integral_constant<int, 0>{});
            if (c + 1 < nchunks) lstep(c + 1, std::integral_constant<int, 1>{});
        }
        __syncthreads();
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
    // Loads go out two steps ahead, into the register set of their step's parity. (The output stores share the
    // vector-memory counter with those loads and the compiler does not count on loads and stores completing in
    // issue order, so the wait before a step's LDS writes covers the loads issued one step before as well.
    // Moving the stores, or keeping one register set, measured slower.)
    const std::integral_constant<bool, true> withq;
    if (nchunks > 0) issue(0, std::integral_constant<int, 0>{}, withq);
    if (nchunks > 1) issue(1, std::integral_constant<int, 1>{}, withq);
    if (chained) {
        f32x4_t Rin[NR];
        chain_enter<NR, NT, true>(ch, seg, anseg, gpow(lg, (float)aseg_len), R, Rin, s_word);
        if (seg > 0 || !a.state_in) {
#pragma unroll
            for (int x = 0; x < NR; ++x) R[x] = Rin[x];
        }
    }
    // decay factors: the mask gamma^(j - l) of this wave's score tile (wave 0: queries 0-15 x keys 0-15, wave
    // 1: queries 16-31 x keys 0-15, wave 2: queries 16-31 x keys 16-31; wave 3 has none), xi_j = gamma^(j+1)
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
    for (int i = tid; i < C * F::LDP; i += NT) sP[i] = 0;  // keys above the diagonal stay zero
    // output row x * 16 + n16 of a step: at row x * 16 + n16 of its rows in memory, or reversed at
    // (1 - x) * 16 + 15 - n16
    const int o_voff = ((REV ? 15 - n16 : n16) * rsv + w * 2 * 16 + g4) * osz;
    auto store_out = [&](int c, const f32x4_t* O) __attribute__((always_inline)) {
        const int L = min(C, seg_n - c * C);
        const rsrc_t ro = bytes_rsrc(oh + crow(c) * rsv * osz, ((L - 1) * rsv + F::DVT) * osz);
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
    // Step c: commit its registers to buffer c & 1 (last read by step c - 2, which every wave finished before
    // step c - 1's first barrier), the loads of step c + 2, barrier, products, P of the score tiles to LDS (sP was
    // last read by step c - 1, which every wave finished before step c's first barrier), barrier, P.V and the
    // output stores.
    auto fstep = [&](int c, auto parc) __attribute__((always_inline)) {
        if (need_rescale(C)) rescale();
        commit(c, parc, withq);
        if (c + 2 < nchunks) issue(c + 2, parc, withq);
        __syncthreads();
        const int buf = c & 1;
        const uint16_t* sQ = smem + buf * F::BUF;
        const uint16_t* sK = sQ + F::SQ;
        const uint16_t* sV = sK + F::SQ;
        const int L = min(C, seg_n - c * C);
        const float gT = gpow(lg, T);  // scale of the state entering the step
        // One pass over d_k in steps of 32: the cross term O^T = R^T Q'^T (the state entering the step,
        // unscaled), this wave's score tile, and the state update of the two d_k blocks the cross term has just
        // read, R^ <- R^ + K'^T (V (.) zeta'). Hand-pipelined: step s + 1's five fragments are read during step
        // s's nine products, and a scheduling fence after each step keeps the compiler from hoisting further.
        const uint16_t* sVz = sV + F::SV;
        f32x4_t O[4], S = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int x = 0; x < 4; ++x) O[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        bf16x8_t fvz[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) fvz[j] = frag_trps<F::DVT>(sVz, 0, (w * 2 + j) * 16, lv_t);
        constexpr int PD = 1;  // steps of fragments read ahead
        bf16x8_t pq[PD][2], pkf[PD], pka[PD][2];
        auto fetch = [&](int s2, int slot) __attribute__((always_inline)) {
            pq[slot][0] = frag_ps<DK>(sQ, 0, 32 * s2, lq_p);
            pq[slot][1] = frag_ps<DK>(sQ, 16, 32 * s2, lq_p);
            pkf[slot] = w < 3 ? frag_ps<DK>(sK, slb * 16, 32 * s2, lq_p) : pq[slot][0];
            pka[slot][0] = frag_trps<DK>(sK, 0, (2 * s2) * 16, lq_t);
            pka[slot][1] = frag_trps<DK>(sK, 0, (2 * s2 + 1) * 16, lq_t);
        };
#pragma unroll
        for (int s2 = 0; s2 < PD; ++s2) fetch(s2, s2);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int slot = s % PD;
            const bf16x8_t q0 = pq[slot][0], q1 = pq[slot][1], kf = pkf[slot], ka0 = pka[slot][0],
                           ka1 = pka[slot][1];
            if (s + PD < KS) fetch(s + PD, slot);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bf16x8_t ra = acc_pair(R[(2 * s) * 2 + j], R[(2 * s + 1) * 2 + j]);
                mfma(O[0 * 2 + j], ra, q0);
                mfma(O[1 * 2 + j], ra, q1);
            }
            if (w < 3) mfma(S, kf, sjb == 0 ? q0 : q1);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                mfma(R[(2 * s) * 2 + j], ka0, fvz[j]);
                mfma(R[(2 * s + 1) * 2 + j], ka1, fvz[j]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        T += (float)L;
        if (w < 3) store4(sP + (sjb * 16 + n16) * F::LDP + slb * 16 + g4, S * DmS);
        __syncthreads();
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
    };
    for (int c = 0; c < nchunks; c += 2) {
        fstep(c, std::integral_constant<int, 0>{});
        if (c + 1 < nchunks) fstep(c + 1, std::integral_constant<int, 1>{});
    }

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
