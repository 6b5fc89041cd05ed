// bf16 single-pass chunkwise kernel for short segments (d_k <= 64, at most 256 tokens per segment): every
// workgroup reads its segment's q, k and v from HBM once and keeps them on chip between the local pass
// (which produces the segment's aggregate for the chain) and the full pass (which produces the outputs).
// Same computation, chain and output layout as chunk_fused_bf16; what differs is where the segment's rows
// live while the workgroup waits for its entering state:
//  * K' (rotated k) of every chunk in its own LDS tile, row-major, read by the score and state-update products;
//  * V as MFMA fragments in registers: wave w only ever reads d_v columns 16w..16w+15 of V, as the A operand of
//    V^T P^T and, scaled by zeta, as the B operand of the state update, so the fragments are formed once (via
//    the LDS tiles that later hold Q') and kept;
//  * Q' (rotated q) in its own LDS tile per chunk, written once the entering state is known (q is read from
//    HBM after k and v, so its loads overlap the chain instead of delaying the local pass).
// Every chunk has its own tiles, so each pass needs one barrier, not one per chunk.
#pragma once

#include "chunk_bf16.h"

namespace ret {

template <int DK, int C, bool PRE>
struct SegB {
    static constexpr int RT = 256;       // tokens of a segment held on chip
    static constexpr int MAXC = RT / C;  // chunks of a segment
    static constexpr int LD = 72;        // row pitch of the Q', K' and V tiles: 36 words mod 64 LDS banks
    static constexpr int NB = C / 16, NKB = DK / 16, KF = C / 32;
    static constexpr int NS = Tri<NB>::count;
    typedef RowTile<C, DK> TQ;  // q and k rows of a chunk
    typedef RowTile<C, 64> TV;  // v rows of the d_v tile
    static constexpr int TILE = C * LD;
    // K' tiles of the segment, then its Q' tiles (which stage V in the local pass)
    static constexpr int LDS_BYTES = 2 * MAXC * TILE * 2;
    static_assert(DK == 32 || DK == 64, "one d_k slice of at most 64");
    static_assert(C == 32 || C == 64, "chunk tile of 32 or 64 tokens");
    static_assert(LDS_BYTES <= 80 * 1024, "two workgroups per CU");
    static_assert((LD / 2) % 64 == 36, "LDS row pitch");
};

template <int DK, int C, bool PRE>
__global__ __launch_bounds__(kThreads, 2) void chunk_seg_bf16(FwdArgs a) {
    typedef SegB<DK, C, PRE> F;
    typedef typename F::TQ TQ;
    typedef typename F::TV TV;
    constexpr int LD = F::LD, KF = F::KF;
    __shared__ __attribute__((aligned(16))) uint16_t smem[F::LDS_BYTES / 2];
    __shared__ int s_word;                            // broadcast word (ticket, finish count)
    // theta in LDS: rotation factors are evaluated while q, k or v loads are in flight, and a wave's vector
    // loads complete in order, so reading theta from global memory then would wait for all of them
    __shared__ double s_theta[DK / 2];
    uint16_t* const sKres = smem;                     // K' of chunk c at sKres + c * TILE
    uint16_t* const sQres = smem + F::MAXC * F::TILE;  // Q' (first V) of chunk c at sQres + c * TILE

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g4 = 4 * (lane >> 4), n16 = lane & 15;
    const int ntiles = __builtin_amdgcn_readfirstlane(a.dv / 64);
    const int units = __builtin_amdgcn_readfirstlane(a.B * a.H * ntiles);
    const int unit = unit_of_block(ntiles, units);
    const Chain ch = chain_of(a.ws, units, a.nseg, unit, DK * 64);
    // Scalar arguments as wave-uniform values.
    const int aN = __builtin_amdgcn_readfirstlane(a.N), aH = __builtin_amdgcn_readfirstlane(a.H);
    const int adk = __builtin_amdgcn_readfirstlane(a.dk), adv = __builtin_amdgcn_readfirstlane(a.dv);
    const int anseg = __builtin_amdgcn_readfirstlane(a.nseg), aseg_len = __builtin_amdgcn_readfirstlane(a.seg_len);
    const int pair = unit / ntiles;
    const int b = pair / aH, h = pair % aH;
    const int dv0 = (unit % ntiles) * 64;
    const float lg = a.log2g[h];
    const int rsk = aH * adk, rsv = aH * adv;  // elements between consecutive tokens
    const int qrow = tid / TQ::SPR, qseg = tid % TQ::SPR;
    const int qoff = (qrow * rsk + qseg * 8) * 2;
    const int vrow = tid / TV::SPR, vseg = tid % TV::SPR;
    const int voff = (vrow * rsv + vseg * 8) * 2;

    // Where segment sg's rows are. A chunk's buffer resources cover its live rows only: rows past the
    // sequence, and every row of a chunk past the segment (an empty resource), read as zero. So loads and tile
    // stores run for every chunk slot with no branch around them, and the waits on them stay exact.
    struct Geom {
        long long t0;  // first token
        int n;         // tokens
        const uint16_t *q, *k, *v;
    };
    auto geom = [&](int sg) __attribute__((always_inline)) {
        Geom g;
        g.t0 = (long long)sg * aseg_len;
        g.n = (int)(min((long long)aN, g.t0 + aseg_len) - g.t0);
        const long long head0 = ((long long)b * aN + g.t0) * aH + h;
        g.q = (const uint16_t*)(PRE ? a.qr : a.q) + head0 * adk;
        g.k = (const uint16_t*)(PRE ? a.kr : a.k) + head0 * adk;
        g.v = (const uint16_t*)a.v + head0 * adv + dv0;
        return g;
    };
    auto rows_rsrc = [&](const Geom& g, const uint16_t* base, int c, int rs, int width) __attribute__((always_inline)) {
        const int L = min(C, g.n - c * C);
        return bytes_rsrc(base + (long long)c * C * rs, L > 0 ? ((L - 1) * rs + width) * 2 : 0);
    };
    u32x4_t rq[F::MAXC][TQ::NP], rk[F::MAXC][TQ::NP], rv[F::MAXC][TV::NP];
    auto issue_kv = [&](const Geom& g) __attribute__((always_inline)) {
        static_for<0, F::MAXC>([&](auto cc) __attribute__((always_inline)) {
            constexpr int c = decltype(cc)::value;
            const rsrc_t bk = rows_rsrc(g, g.k, c, rsk, DK), bv = rows_rsrc(g, g.v, c, rsv, 64);
#pragma unroll
            for (int p = 0; p < TQ::NP; ++p) rk[c][p] = buf_load16(bk, qoff, p * TQ::RP * rsk * 2);
#pragma unroll
            for (int p = 0; p < TV::NP; ++p) rv[c][p] = buf_load16(bv, voff, p * TV::RP * rsv * 2);
        });
    };
    constexpr int NQLOADS = F::MAXC * TQ::NP;  // vector memory operations of issue_q per thread
    auto issue_q = [&](const Geom& g) __attribute__((always_inline)) {
        static_for<0, F::MAXC>([&](auto cc) __attribute__((always_inline)) {
            constexpr int c = decltype(cc)::value;
            const rsrc_t bq = rows_rsrc(g, g.q, c, rsk, DK);
#pragma unroll
            for (int p = 0; p < TQ::NP; ++p) rq[c][p] = buf_load16(bq, qoff, p * TQ::RP * rsk * 2);
        });
    };

    // ---- the segment: the unit's next ticket (so every earlier segment of the unit has started); then its k
    // and v rows, all issued at once. ----
    if constexpr (!PRE)
        if (tid < DK / 2) s_theta[tid] = a.theta[tid];  // visible after the ticket's barriers
    const int seg = chain_ticket(ch, s_word);
    issue_kv(geom(seg));
    issue_q(geom(seg));
    const Geom G = geom(seg);
    const long long seg_t0 = G.t0;
    const int seg_n = G.n;
    const int nchunks = (seg_n + C - 1) / C;  // at most MAXC: the host plans segments of at most RT tokens
    const int osz = a.out_bf16 ? 2 : 4;
    char* oh = (char*)a.o + ((((long long)b * aN + seg_t0) * aH + h) * adv + dv0) * osz;
    const bool last = seg == anseg - 1;
    const bool boundary = seg % kChainGroup == kChainGroup - 1;
    const int tro = trp_lane_offset(LD, lane);

    f32x4_t R[F::NKB];
#pragma unroll
    for (int x = 0; x < F::NKB; ++x) R[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // State_in enters through the first segment: its aggregate starts from it (so every later R_in carries
    // it) and its full pass starts from it again.
    auto load_state_in = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < F::NKB; ++x)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                R[x][e] = a.state_in[((long long)pair * DK + x * 16 + g4 + e) * adv + dv0 + w * 16 + n16];
    };
    if (seg == 0 && a.state_in) load_state_in();

    // zeta_t = gamma^(C-1-t) of the tokens a lane holds in a V^T fragment of a full chunk: in the permuted
    // order, tokens 32f + g4 + i and 32f + 16 + g4 + i.
    float zf[KF][8];
#pragma unroll
    for (int f = 0; f < KF; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            zf[f][i] = gpow(lg, (float)(C - 1 - (32 * f + g4 + i)));
            zf[f][4 + i] = gpow(lg, (float)(C - 1 - (32 * f + 16 + g4 + i)));
        }
    const float gC = gpow(lg, (float)C);

    // V fragments of the segment: fv[c][f] is the V^T operand of chunk c, tokens 32f.. (permuted order), and
    // fvz[c][f] the same scaled by zeta (a full chunk's, or the tail chunk's: 0 past its end).
    bf16x8_t fv[F::MAXC][KF], fvz[F::MAXC][KF];
    auto make_fvz = [&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        const int L = min(C, seg_n - c * C);
        float z[KF][8];
        if (L >= C) {
#pragma unroll
            for (int f = 0; f < KF; ++f)
#pragma unroll
                for (int e = 0; e < 8; ++e) z[f][e] = zf[f][e];
        } else {
#pragma unroll
            for (int f = 0; f < KF; ++f)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int t = 32 * f + (e < 4 ? g4 + e : 16 + g4 + e - 4);
                    z[f][e] = t < L ? gpow(lg, (float)(L - 1 - t)) : 0.f;
                }
        }
#pragma unroll
        for (int f = 0; f < KF; ++f) {
            float vf[8];
            unpack8(__builtin_bit_cast(u32x4_t, fv[c][f]), vf);
#pragma unroll
            for (int e = 0; e < 8; ++e) vf[e] *= z[f][e];
            fvz[c][f] = __builtin_bit_cast(bf16x8_t, pack8(vf));
        }
    };
    // R <- gamma^L R + K'^T (V (.) zeta) over chunk c.
    auto update = [&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        const int L = min(C, seg_n - c * C);
        const float gL = L == C ? gC : gpow(lg, (float)L);
        const uint16_t* sK = sKres + c * F::TILE;
#pragma unroll
        for (int x = 0; x < F::NKB; ++x) R[x] *= gL;
#pragma unroll
        for (int f = 0; f < KF; ++f)
#pragma unroll
            for (int x = 0; x < F::NKB; ++x) mfma(R[x], frag_trp(sK, LD, 32 * f, x * 16, tro), fvz[c][f]);
    };

    // ---- local pass: K' into its tiles and V into the Q' tiles as each chunk arrives, then (one barrier)
    // the V fragments and, except in the last segment (whose aggregate no one reads), the aggregate ----
    // Rotation factors of the thread's rows (identity without rotation: theta all zero). Evaluated exactly
    // every 8 chunks, by angle addition in between; the q rows later take the same sequence of factors.
    auto rotate_rows = [&](u32x4_t (*rows)[TQ::NP], uint16_t* tiles) __attribute__((always_inline)) {
        SliceRot<C, TQ::RP, TQ::NP> rot;
        if constexpr (!PRE) rot.init_steps(s_theta, qseg * 4);
        static_for<0, F::MAXC>([&](auto cc) __attribute__((always_inline)) {
            constexpr int c = decltype(cc)::value;
            uint16_t* t = tiles + c * F::TILE;
            if constexpr (!PRE)
                if (c % 8 == 0) rot.cur.eval(a.pos0 + seg_t0 + (long long)c * C + qrow, s_theta, qseg * 4);
#pragma unroll
            for (int p = 0; p < TQ::NP; ++p)
                if (TQ::live(qrow, p)) {
                    if constexpr (PRE) {
                        lds_store16(t + (qrow + p * TQ::RP) * LD + qseg * 8, rows[c][p]);
                    } else {
                        float xf[8];
                        unpack8(rows[c][p], xf);
                        rot.cur.apply(xf);
                        if (p + 1 < TQ::NP) rot.cur.turn(rot.pass);
                        lds_store16(t + (qrow + p * TQ::RP) * LD + qseg * 8, pack8(xf));
                    }
                }
            if constexpr (!PRE) rot.next_chunk();
        });
    };
    rotate_rows(rk, sKres);
    static_for<0, F::MAXC>([&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
#pragma unroll
        for (int p = 0; p < TV::NP; ++p)
            if (TV::live(vrow, p)) lds_store16(sQres + c * F::TILE + (vrow + p * TV::RP) * LD + vseg * 8, rv[c][p]);
    });
    __syncthreads();
    static_for<0, F::MAXC>([&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        if (c < nchunks) {
#pragma unroll
            for (int f = 0; f < KF; ++f) fv[c][f] = frag_trp(sQres + c * F::TILE, LD, 32 * f, w * 16, tro);
            make_fvz(cc);
            if (!last) update(cc);
        }
    });

    // ---- segment chain: publish the aggregate, then the entering state ----
    if (!last && !boundary) chain_publish<F::NKB>(ch, seg, R);
    {
        f32x4_t Rin[F::NKB];
        chain_enter<F::NKB, false>(ch, seg, anseg, gpow(lg, (float)aseg_len), R, Rin, s_word);
#pragma unroll
        for (int x = 0; x < F::NKB; ++x) R[x] = Rin[x];
        if (seg == 0) {
#pragma unroll
            for (int x = 0; x < F::NKB; ++x) R[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (a.state_in) load_state_in();
        }
    }

    // ---- full pass from on-chip operands ----
    // The mask gamma^(j-l) for S^T tiles Delta = jb - lb blocks below the diagonal (rows l, columns j of the
    // lane) and xi_j = gamma^(j+1) of each O^T tile (column j).
    float Dm[F::NB][4], Xi[F::NB];
#pragma unroll
    for (int d = 0; d < F::NB; ++d)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int jl = 16 * d + n16 - g4 - e;  // j - l
            Dm[d][e] = jl >= 0 ? gpow(lg, (float)jl) : 0.f;
        }
#pragma unroll
    for (int x = 0; x < F::NB; ++x) Xi[x] = gpow(lg, (float)(x * 16 + n16 + 1));

    // Output stores straight from the O^T accumulators: lane (g, n16) of tile x holds 4 consecutive d_v of
    // query x*16 + n16. Rows past the sequence fall outside the buffer range and are dropped.
    const int o_voff = (n16 * rsv + w * 16 + g4) * osz;
    auto store_out = [&](int c, const f32x4_t* O) __attribute__((always_inline)) {
        const int L = min(C, seg_n - c * C);
        const rsrc_t ro = bytes_rsrc(oh + (long long)c * C * rsv * osz, ((L - 1) * rsv + 64) * osz);
        if (a.out_bf16) {
#pragma unroll
            for (int x = 0; x < F::NB; ++x)
                __builtin_amdgcn_raw_buffer_store_b64(
                    __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(2))),
                                       make_uint2(pack2_bf16(O[x][0], O[x][1]), pack2_bf16(O[x][2], O[x][3]))),
                    ro, o_voff, x * 16 * rsv * 2, kOutAux);
        } else {
#pragma unroll
            for (int x = 0; x < F::NB; ++x)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, O[x]), ro, o_voff, x * 16 * rsv * 4,
                                                       kOutAux);
        }
    };
    auto tri = [](int jb, int lb) constexpr { return jb * (jb + 1) / 2 + lb; };

    // Q' into the tiles that staged V (every wave read its V fragments before the chain's barriers); then the
    // chunks need no barrier: their operands are all on chip and only the state carries from one to the next.
    rotate_rows(rq, sQres);
    __syncthreads();
    static_for<0, F::MAXC>([&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        if (c < nchunks) {
            const uint16_t* sQ = sQres + c * F::TILE;
            const uint16_t* sK = sKres + c * F::TILE;
            f32x4_t S[F::NS], O[F::NB];
#pragma unroll
            for (int x = 0; x < F::NS; ++x) S[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int x = 0; x < F::NB; ++x) O[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            // S^T = K' Q'^T (every lower-triangle tile: each wave needs all of P) and the cross term
            // O^T = R^T Q'^T, R^T taken from the state accumulators (the state entering this chunk).
#pragma unroll
            for (int kk = 0; kk < DK; kk += 32) {
                bf16x8_t qf[F::NB], kf[F::NB];
#pragma unroll
                for (int x = 0; x < F::NB; ++x) {
                    qf[x] = frag_p(sQ + x * 16 * LD, LD, kk, lane);
                    kf[x] = frag_p(sK + x * 16 * LD, LD, kk, lane);
                }
#pragma unroll
                for (int jb = 0; jb < F::NB; ++jb)
#pragma unroll
                    for (int lb = 0; lb <= jb; ++lb) mfma(S[tri(jb, lb)], kf[lb], qf[jb]);
                const bf16x8_t ra = acc_pair(R[kk / 16], R[kk / 16 + 1]);
#pragma unroll
                for (int x = 0; x < F::NB; ++x) mfma(O[x], ra, qf[x]);
            }
            update(cc);
            // O^T = xi (.) O^T + V^T P^T, P = mask (.) S from the S^T accumulators as the B operand (keys 32f..
            // of query block x are tiles lb = 2f and 2f + 1).
#pragma unroll
            for (int x = 0; x < F::NB; ++x) O[x] *= Xi[x];
#pragma unroll
            for (int f = 0; f < KF; ++f) {
#pragma unroll
                for (int x = 2 * f; x < F::NB; ++x) {
                    const f32x4_t p0 = S[tri(x, 2 * f)] * f32x4_t{Dm[x - 2 * f][0], Dm[x - 2 * f][1],
                                                                  Dm[x - 2 * f][2], Dm[x - 2 * f][3]};
                    f32x4_t p1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    if (2 * f + 1 <= x)
                        p1 = S[tri(x, 2 * f + 1)] * f32x4_t{Dm[x - 2 * f - 1][0], Dm[x - 2 * f - 1][1],
                                                            Dm[x - 2 * f - 1][2], Dm[x - 2 * f - 1][3]};
                    mfma(O[x], fv[c][f], acc_pair(p0, p1));
                }
            }
            store_out(c, O);
        }
    });

    // The state after the last token of the sequence.
    if (last && a.state_out) {
        float* out = a.state_out + (long long)pair * DK * adv;
#pragma unroll
        for (int x = 0; x < F::NKB; ++x) {
#pragma unroll
            for (int e = 0; e < 4; ++e) out[(long long)(x * 16 + g4 + e) * adv + dv0 + w * 16 + n16] = R[x][e];
        }
    }
    chain_finish(a, 64, DK * 64, s_word);
}

}  // namespace ret
