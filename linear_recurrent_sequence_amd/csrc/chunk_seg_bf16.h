// bf16 single-pass chunkwise kernel for short segments (d_k <= 64, at most 256 tokens per segment). Each
// workgroup streams its segment once, running the chunkwise form from the state it knows without the chain
// (zero, or state_in for the first segment), while the segment's rows arrive. The state entering chunk c of
// the segment is gamma^(cC) R_in + R_c, where R_c is that local state and R_in the state entering the segment
// (chunkwise recurrence; the chain supplies R_in). So the outputs differ from the local ones only by the
// cross term of R_in,
//     O_c = O_c(local) + xi (.) gamma^(cC) (Q'_c R_in),
// which is added once R_in is known. Until then each chunk's local outputs stay in fp32 registers and its Q'
// (rotated q) stays in its own LDS tile; the local end state is the segment's aggregate, published for the
// later segments as soon as the last chunk is done. The chain's latency thus overlaps the segment's streaming
// and main products instead of preceding them, and q, k and v are read from HBM once (with the non-temporal
// hint: no row is read again).
//
// REV runs the same recurrence over the reversed sequence (token n of the run is row N-1-n of q, k, v and o):
// the gradients' retentions that sum over later tokens, without state in, state out or the epilogue. Every row
// of a reversed chunk gets its own buffer offset, which is negative, hence out of range and read as zero or
// dropped, for rows past the chunk. Rows are rotated (q and k without PRE; v with a.vrot, PRE and GR) by the
// rotation at their own positions in memory.
#pragma once

#include "chunk_bf16.h"

namespace ret {

template <int DK, int C, bool PRE>
struct SegB {
    static constexpr int RT = 256;       // tokens of a segment held on chip
    static constexpr int MAXC = RT / C;  // chunks of a segment
    // Q' tiles are read as row fragments only: a row pitch of 36 words mod 64 LDS banks serves them. The K'
    // and V staging tiles, read transposed as well, are Swz tiles.
    static constexpr int LD = 72;
    static constexpr int NB = C / 16, NKB = DK / 16, KF = C / 32, KK = DK / 32;
    static constexpr int NBUF = 2;       // chunks of loads in flight ahead of the one being staged
    typedef RowTile<C, DK> TQ;           // q and k rows of a chunk
    typedef RowTile<C, 64> TV;           // v rows of the d_v tile
    static constexpr int TILE = C * LD, KTILE = C * Swz<DK>::LD, VTILE = C * Swz<64>::LD;
    // Q' tiles of the segment, then two K' and two V staging tiles
    static constexpr int LDS_BYTES = (MAXC * TILE + 2 * KTILE + 2 * VTILE) * 2;
    static_assert(DK == 32 || DK == 64, "one d_k slice of at most 64");
    static_assert(C == 32 || C == 64, "chunk tile of 32 or 64 tokens");
    static_assert(LDS_BYTES <= 80 * 1024, "two workgroups per CU");
    static_assert((LD / 2) % 64 == 36, "LDS row pitch");
    static_assert(VTILE >= TILE, "a V staging tile holds a chunk of bf16 output rows at pitch LD");
};

template <int DK, int C, bool PRE, bool REV = false, bool GR = false>
__global__ __launch_bounds__(kThreads, 2) void chunk_seg_bf16(FwdArgs a) {
    typedef SegB<DK, C, PRE> F;
    typedef typename F::TQ TQ;
    typedef typename F::TV TV;
    constexpr int LD = F::LD, KF = F::KF, NB = F::NB, KK = F::KK, NBUF = F::NBUF;
    __shared__ __attribute__((aligned(16))) uint16_t smem[F::LDS_BYTES / 2];
    __shared__ int s_word;  // broadcast word (ticket, finish count)
    // theta in LDS: rotation factors are evaluated while loads are in flight, and reading theta from global
    // memory then would wait behind them
    __shared__ double s_theta[DK / 2];
    uint16_t* const sQres = smem;                     // Q' of chunk c at sQres + c * TILE
    uint16_t* const sKst = smem + F::MAXC * F::TILE;  // K' staging tiles 0, 1
    uint16_t* const sVst = sKst + 2 * F::KTILE;       // V staging tiles 0, 1
    typedef Swz<DK> ZK;
    typedef Swz<64> ZV;

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g4 = 4 * (lane >> 4), n16 = lane & 15;
    const int ntiles = __builtin_amdgcn_readfirstlane(a.dv / 64);
    const int units = __builtin_amdgcn_readfirstlane(a.B * a.H * ntiles);
    const int unit = unit_of_block(ntiles, units);
    const Chain ch = chain_of(a.ws, units, a.nseg, unit, DK * 64, a.chain_spin);
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
    const int lk_p = ZK::lane_p(lane), lk_t = ZK::lane_trp(lane), lv_t = ZV::lane_trp(lane);

    // ---- the segment: the unit's next ticket, so every earlier segment of the unit has started ----
    if constexpr (!PRE)
        if (tid < DK / 2) s_theta[tid] = a.theta[tid];  // visible after the ticket's barriers
    // The segment is the unit's next ticket, known only after a device-scope atomic. The first chunks' loads go
    // out before it for the segment of the launch order (the usual ticket), and again if the ticket differs.
    int seg = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / (unsigned)units));
    long long seg_t0, head0;
    int seg_n, nchunks;
    const uint16_t *qh, *kh, *vh;
    char* oh;
    const int osz = a.out_bf16 ? 2 : 4;
    auto place = [&](int sg) __attribute__((always_inline)) {
        seg_t0 = (long long)sg * aseg_len;
        seg_n = (int)(min((long long)aN, seg_t0 + aseg_len) - seg_t0);  // tokens in this segment
        nchunks = (seg_n + C - 1) / C;  // at most MAXC: the host plans segments of at most RT tokens
        // REV: the rows of the run's chunk c start (in memory order) at token N - seg_t0 - c*C - L, so the head
        // pointers address token 0 and rows_tok0 adds the chunk's first row.
        head0 = ((long long)b * aN + (REV ? 0 : seg_t0)) * aH + h;
        qh = (const uint16_t*)(PRE ? a.qr : a.q) + head0 * adk;
        kh = (const uint16_t*)(PRE ? a.kr : a.k) + head0 * adk;
        vh = (const uint16_t*)a.v + head0 * adv + dv0;
        oh = (char*)a.o + (head0 * adv + dv0) * osz;
    };
    place(seg);

    // ---- loads: q, k and v rows of chunk c into register buffer c % NBUF. A chunk's buffer resources cover
    // its live rows only: rows past the sequence, and every row of a chunk past the segment (an empty
    // resource), read as zero, so loads and tile stores need no branch and the waits on them stay exact. ----
    // first row of chunk c in memory (in rows after the head pointer), and the byte offset of its row r: rows
    // past the chunk's L live rows get a negative offset under REV, out of every range
    auto rows_tok0 = [&](int c, int L) __attribute__((always_inline)) {
        return REV ? (long long)aN - seg_t0 - (long long)c * C - L : (long long)c * C;
    };
    auto row_off = [&](int L, int r, int rs, int col, int esz) __attribute__((always_inline)) {
        return ((REV ? L - 1 - r : r) * rs + col) * esz;
    };
    auto rows_rsrc = [&](const uint16_t* base, int c, int rs, int width) __attribute__((always_inline)) {
        const int L = min(C, seg_n - c * C);
        return bytes_rsrc(base + rows_tok0(c, L) * rs, L > 0 ? ((L - 1) * rs + width) * 2 : 0);
    };
    u32x4_t bq[NBUF][TQ::NP], bk[NBUF][TQ::NP], bv[NBUF][TV::NP];
    auto issue = [&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value, par = c % NBUF;
        const rsrc_t rq = rows_rsrc(qh, c, rsk, DK), rk = rows_rsrc(kh, c, rsk, DK), rv = rows_rsrc(vh, c, rsv, 64);
        if constexpr (REV) {
            const int L = min(C, seg_n - c * C);
#pragma unroll
            for (int p = 0; p < TQ::NP; ++p) {
                const int off = row_off(L, qrow + p * TQ::RP, rsk, qseg * 8, 2);
                bk[par][p] = buf_load16_nt(rk, off, 0);
                bq[par][p] = buf_load16_nt(rq, off, 0);
            }
#pragma unroll
            for (int p = 0; p < TV::NP; ++p) bv[par][p] = buf_load16_nt(rv, row_off(L, vrow + p * TV::RP, rsv, vseg * 8, 2), 0);
        } else {
#pragma unroll
            for (int p = 0; p < TQ::NP; ++p) {
                bk[par][p] = buf_load16_nt(rk, qoff, p * TQ::RP * rsk * 2);
                bq[par][p] = buf_load16_nt(rq, qoff, p * TQ::RP * rsk * 2);
            }
#pragma unroll
            for (int p = 0; p < TV::NP; ++p) bv[par][p] = buf_load16_nt(rv, voff, p * TV::RP * rsv * 2);
        }
    };
    static_for<0, (NBUF < F::MAXC ? NBUF : F::MAXC)>([&](auto cc) __attribute__((always_inline)) { issue(cc); });
    {
        const int tk = chain_ticket(ch, s_word);
        if (tk != seg) {
            seg = tk;
            place(seg);
            static_for<0, (NBUF < F::MAXC ? NBUF : F::MAXC)>([&](auto cc) __attribute__((always_inline)) { issue(cc); });
        }
    }
    const bool last = seg == anseg - 1;
    const bool boundary = seg % kChainGroup == kChainGroup - 1;

    // The local state: zero, or state_in for the first segment (which then needs no chain term).
    f32x4_t R[F::NKB];
#pragma unroll
    for (int x = 0; x < F::NKB; ++x) R[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (seg == 0 && a.state_in) {
#pragma unroll
        for (int x = 0; x < F::NKB; ++x)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                R[x][e] = a.state_in[((long long)pair * DK + x * 16 + g4 + e) * adv + dv0 + w * 16 + n16];
    }

    // Chunk-independent factors: the mask gamma^(j-l) for S^T tiles Delta = jb - lb blocks below the diagonal
    // (rows l, columns j of the lane) and xi_j = gamma^(j+1) of each O^T tile (column j).
    float Dm[NB][4], Xi[NB];
#pragma unroll
    for (int d = 0; d < NB; ++d)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int jl = 16 * d + n16 - g4 - e;  // j - l
            Dm[d][e] = jl >= 0 ? gpow(lg, (float)jl) : 0.f;
        }
#pragma unroll
    for (int x = 0; x < NB; ++x) Xi[x] = gpow(lg, (float)(x * 16 + n16 + 1));
    const float gC = gpow(lg, (float)C);

    // Rotation factors of the thread's rows (identity without rotation: theta all zero), shared by its q and k
    // rows. Evaluated exactly every 8 chunks, by angle addition in between. Run row r of chunk c is at position
    // pos0 + seg_t0 + cC + r, or over the reversed sequence pos0 + N - 1 - (seg_t0 + cC + r).
    SliceRot<C, TQ::RP, TQ::NP, REV ? 2 : 0> rot;
    if constexpr (!PRE) rot.init_steps(s_theta, qseg * 4);
    auto run_pos = [&](int c, int r) __attribute__((always_inline)) {
        const long long t = seg_t0 + (long long)c * C + r;
        return a.pos0 + (REV ? (long long)aN - 1 - t : t);
    };
    // PRE with GR and a.vrot: the factors of the thread's v rows (columns dv0 + 8 vseg ..), the same way
    constexpr bool VR = PRE && GR;
    SliceRot<C, TV::RP, TV::NP, REV ? 2 : 0> vrt;
    const int vpair0 = (dv0 + vseg * 8) / 2;
    if constexpr (VR)
        if (a.vrot) vrt.init_steps(a.theta, vpair0);

    // Output stores straight from the O^T accumulators: lane (g, n16) of tile x holds 4 consecutive d_v of
    // query x*16 + n16. Rows past the sequence fall outside the buffer range and are dropped.
    const int o_voff = (n16 * rsv + w * 16 + g4) * osz;
    auto store_out = [&](int c, const f32x4_t* O) __attribute__((always_inline)) {
        const int L = min(C, seg_n - c * C);
        const rsrc_t ro = bytes_rsrc(oh + rows_tok0(c, L) * rsv * osz, ((L - 1) * rsv + 64) * osz);
        // REV: row x*16 + n16 at its own (possibly negative) offset; else one offset plus a scalar per tile
        const int vo = REV ? row_off(L, n16, rsv, w * 16 + g4, osz) : o_voff;
        if (a.out_bf16) {
#pragma unroll
            for (int x = 0; x < NB; ++x)
                __builtin_amdgcn_raw_buffer_store_b64(
                    __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(2))),
                                       make_uint2(pack2_bf16(O[x][0], O[x][1]), pack2_bf16(O[x][2], O[x][3]))),
                    ro, REV ? vo - x * 16 * rsv * 2 : vo, REV ? 0 : x * 16 * rsv * 2, kOutAux);
        } else {
#pragma unroll
            for (int x = 0; x < NB; ++x)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, O[x]), ro,
                                                       REV ? vo - x * 16 * rsv * 4 : vo, REV ? 0 : x * 16 * rsv * 4,
                                                       kOutAux);
        }
    };

    // ---- one pass over the segment's chunks from the local state ----
    f32x4_t Op[F::MAXC][NB];  // local outputs O^T of each chunk (fp32) until the chain's term is added
    static_for<0, F::MAXC>([&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value, par = c % NBUF;
        if (c < nchunks) {
            // Stage chunk c: Q' into its own tile, K' and V into staging tile c % 2 (last read by chunk c - 2,
            // whose products every wave finished before the barrier of chunk c - 1).
            uint16_t* sQ = sQres + c * F::TILE;
            uint16_t* sK = sKst + (c & 1) * F::KTILE;
            uint16_t* sV = sVst + (c & 1) * F::VTILE;
            if constexpr (!PRE)
                if (c % 8 == 0) rot.cur.eval(run_pos(c, qrow), s_theta, qseg * 4);
#pragma unroll
            for (int p = 0; p < TQ::NP; ++p)
                if (TQ::live(qrow, p)) {
                    const int r = (qrow + p * TQ::RP) * LD + qseg * 8;
                    const int rk = ZK::off(qrow + p * TQ::RP, qseg * 8);
                    if constexpr (PRE) {
                        lds_store16(sQ + r, bq[par][p]);
                        lds_store16(sK + rk, bk[par][p]);
                    } else {
                        float qf[8], kf[8];
                        unpack8(bq[par][p], qf);
                        unpack8(bk[par][p], kf);
                        rot.cur.apply(qf);
                        rot.cur.apply(kf);
                        if (p + 1 < TQ::NP) rot.cur.turn(rot.pass);
                        lds_store16(sQ + r, pack8(qf));
                        lds_store16(sK + rk, pack8(kf));
                    }
                }
            if constexpr (!PRE) rot.next_chunk();
            if (VR && a.vrot && c % 8 == 0) vrt.cur.eval(run_pos(c, vrow), a.theta, vpair0);
#pragma unroll
            for (int p = 0; p < TV::NP; ++p)
                if (TV::live(vrow, p)) {
                    if (VR && a.vrot) {
                        float vf[8];
                        unpack8(bv[par][p], vf);
                        vrt.cur.apply(vf);
                        if (p + 1 < TV::NP) vrt.cur.turn(vrt.pass);
                        lds_store16(sV + ZV::off(vrow + p * TV::RP, vseg * 8), pack8(vf));
                    } else {
                        lds_store16(sV + ZV::off(vrow + p * TV::RP, vseg * 8), bv[par][p]);
                    }
                }
            if (VR && a.vrot) vrt.next_chunk();
            if constexpr (c + NBUF < F::MAXC) issue(std::integral_constant<int, c + NBUF>{});
            __syncthreads();

            const int L = min(C, seg_n - c * C);
            // V^T fragments of d_v block w (permuted order: tokens 32f + g4 + i and 32f + 16 + g4 + i), and the
            // same scaled by zeta_t = gamma^(L-1-t) (0 past the chunk's end) for the state update.
            bf16x8_t fv[KF], fvz[KF];
#pragma unroll
            for (int f = 0; f < KF; ++f) {
                fv[f] = frag_trps<64>(sV, 32 * f, w * 16, lv_t);
                float vf[8];
                unpack8(__builtin_bit_cast(u32x4_t, fv[f]), vf);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int t = 32 * f + (e < 4 ? g4 + e : 16 + g4 + e - 4);
                    vf[e] *= t < L ? gpow(lg, (float)(L - 1 - t)) : 0.f;
                }
                fvz[f] = __builtin_bit_cast(bf16x8_t, pack8(vf));
            }
            // K' fragments of every key block (rows of S^T) and R^T operands of the cross term (the state
            // entering this chunk, before its update).
            bf16x8_t kf[KK][NB], ra[KK];
#pragma unroll
            for (int k = 0; k < KK; ++k) {
                ra[k] = acc_pair(R[2 * k], R[2 * k + 1]);
#pragma unroll
                for (int lb = 0; lb < NB; ++lb) kf[k][lb] = frag_ps<DK>(sK, lb * 16, 32 * k, lk_p);
            }
            // Per query block x: S^T tiles (x, lb <= x) = K' Q'^T, the cross term O^T = R^T Q'^T, then
            // O^T = xi (.) O^T + V^T P^T with P = mask (.) S from the S^T accumulators as the B operand (keys
            // 32f.. of block x are tiles lb = 2f and 2f + 1).
#pragma unroll
            for (int x = 0; x < NB; ++x) {
                f32x4_t S[NB];
#pragma unroll
                for (int lb = 0; lb <= x; ++lb) S[lb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                f32x4_t O = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < KK; ++k) {
                    const bf16x8_t qf = frag_p(sQ + x * 16 * LD, LD, 32 * k, lane);
#pragma unroll
                    for (int lb = 0; lb <= x; ++lb) mfma(S[lb], kf[k][lb], qf);
                    mfma(O, ra[k], qf);
                }
                O *= Xi[x];
#pragma unroll
                for (int f = 0; 2 * f <= x; ++f) {
                    const f32x4_t p0 = S[2 * f] * f32x4_t{Dm[x - 2 * f][0], Dm[x - 2 * f][1], Dm[x - 2 * f][2],
                                                          Dm[x - 2 * f][3]};
                    f32x4_t p1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    if (2 * f + 1 <= x)
                        p1 = S[2 * f + 1] * f32x4_t{Dm[x - 2 * f - 1][0], Dm[x - 2 * f - 1][1],
                                                    Dm[x - 2 * f - 1][2], Dm[x - 2 * f - 1][3]};
                    mfma(O, fv[f], acc_pair(p0, p1));
                }
                Op[c][x] = O;
            }
            // R <- gamma^L R + K'^T (V (.) zeta)
            const float gL = L == C ? gC : gpow(lg, (float)L);
#pragma unroll
            for (int x = 0; x < F::NKB; ++x) R[x] *= gL;
#pragma unroll
            for (int f = 0; f < KF; ++f)
#pragma unroll
                for (int x = 0; x < F::NKB; ++x) mfma(R[x], frag_trps<DK>(sK, 32 * f, x * 16, lk_t), fvz[f]);
        }
    });

    // ---- segment chain: publish the local end state (the aggregate), then the entering state R_in ----
    if (!last && !boundary) chain_publish<F::NKB, kThreads>(ch, seg, R);
    f32x4_t Rin[F::NKB];
    chain_enter<F::NKB, kThreads, false>(ch, seg, anseg, gpow(lg, (float)aseg_len), R, Rin, s_word);

    // ---- the chain's term, then the outputs: O_c += xi (.) gamma^(cC) (Q'_c R_in) ----
    // bf16 outputs leave through the V staging tiles (free by now; chunk c uses tile c % 2, last read before the
    // barrier of chunk c - 1) as whole rows: each wave writes its O^T tiles as rows of O, then 8 lanes store one
    // row's 64 d_v (128 bytes) with one 16-byte store each, instead of four waves writing 32-byte pieces of it.
    //
    // With the multi-scale retention epilogue (a.epi; d_v = 64, so a row is a whole head) the 8 lanes of a row
    // hold one GroupNorm group: they standardize it by shuffles, apply the per-channel affine and the swish
    // gate, and store y in place of o. The gate rows are read with the same range as the output rows, one chunk
    // ahead of their use (gq[c % 2]), so only the first chunk's read is waited for in full.
    const int gsz = a.gate_bf16 ? 2 : 4;
    const char* gh = (const char*)a.gate + (head0 * adv + dv0) * gsz;
    const int row = tid / 8, sg = tid % 8;
    u32x4_t gq[2][C / 32][2];
    auto gate_issue = [&](int c, u32x4_t (&gu)[C / 32][2]) __attribute__((always_inline)) {
        if (!REV && a.epi && a.gate && c < nchunks) {
            const int L = min(C, seg_n - c * C);
            const rsrc_t rg = bytes_rsrc(gh + (long long)c * C * rsv * gsz, ((L - 1) * rsv + 64) * gsz);
#pragma unroll
            for (int p = 0; p < C / 32; ++p) {
                const int off = ((row + 32 * p) * rsv + sg * 8) * gsz;
                gu[p][0] = buf_load16_nt(rg, off, 0);
                gu[p][1] = a.gate_bf16 ? u32x4_t{0u, 0u, 0u, 0u} : buf_load16_nt(rg, off + 16, 0);
            }
        }
    };
    auto store_rows = [&](int c, const f32x4_t* O, uint16_t* buf, const u32x4_t (&gu)[C / 32][2])
                          __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < NB; ++x)
            *reinterpret_cast<uint2*>(buf + (x * 16 + n16) * LD + w * 16 + g4) =
                make_uint2(pack2_bf16(O[x][0], O[x][1]), pack2_bf16(O[x][2], O[x][3]));
        const int L = min(C, seg_n - c * C);
        __syncthreads();
        const rsrc_t ro = bytes_rsrc(oh + rows_tok0(c, L) * rsv * 2, ((L - 1) * rsv + 64) * 2);
#pragma unroll
        for (int p = 0; p < C / 32; ++p) {
            u32x4_t u = *reinterpret_cast<const u32x4_t*>(buf + (row + 32 * p) * LD + sg * 8);
            if (!REV && a.epi) {
                float x[8];
                unpack8(u, x);
                group_standardize<8, 8>(x, 64.f, a.eps);
                const int ch = h * 64 + sg * 8;
                if (a.gn_weight) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] *= a.gn_weight[ch + e];
                }
                if (a.gn_bias) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] += a.gn_bias[ch + e];
                }
                if (a.gate) {
                    float gv[8];
                    if (a.gate_bf16) {
                        unpack8(gu[p][0], gv);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            gv[e] = __uint_as_float(gu[p][0][e]);
                            gv[4 + e] = __uint_as_float(gu[p][1][e]);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] *= swish_hw(gv[e]);
                }
                u = pack8(x);
            }
            buf_store16(ro, row_off(L, row + 32 * p, rsv, sg * 8, 2), 0, u);
        }
    };
    bf16x8_t rin[KK];
#pragma unroll
    for (int k = 0; k < KK; ++k) rin[k] = acc_pair(Rin[2 * k], Rin[2 * k + 1]);
    // a.orot (PRE only, for the gradients): every output row turned back by the transpose of the rotation at its
    // position. The lane's tile values are columns dv0 + 16w + g4 .. + 3 (two pairs) of run row x*16 + n16; the
    // factors start exactly at the lane's first row and step 16 rows at a time by angle addition.
    float oc[2] = {1.f, 1.f}, os[2] = {0.f, 0.f}, sc[2] = {1.f, 1.f}, ss[2] = {0.f, 0.f};
    if constexpr (PRE) {
        if (a.orot) {
            const int p0 = (dv0 + w * 16 + g4) / 2;
            const long long t0 = seg_t0 + n16;  // run index of the lane's row in tile 0 of chunk 0
            const long long pos = a.pos0 + (REV ? (long long)aN - 1 - t0 : t0);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                rot_cs(pos, a.theta[p0 + j], &oc[j], &os[j]);
                rot_cs(REV ? -16 : 16, a.theta[p0 + j], &sc[j], &ss[j]);
            }
        }
    }
    if (a.out_bf16) gate_issue(0, gq[0]);
    static_for<0, F::MAXC>([&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        if (c < nchunks) {
            if (a.out_bf16 && c + 1 < F::MAXC) gate_issue(c + 1, gq[(c + 1) % 2]);
            if (seg > 0) {
                const uint16_t* sQ = sQres + c * F::TILE;
                const float gc = gpow(lg, (float)(c * C));
#pragma unroll
                for (int x = 0; x < NB; ++x) {
                    f32x4_t X = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < KK; ++k) mfma(X, rin[k], frag_p(sQ + x * 16 * LD, LD, 32 * k, lane));
                    Op[c][x] += (gc * Xi[x]) * X;
                }
            }
            if constexpr (PRE) {
                if (a.orot) {
#pragma unroll
                    for (int x = 0; x < NB; ++x)
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            const float x0 = Op[c][x][2 * j], x1 = Op[c][x][2 * j + 1];
                            Op[c][x][2 * j] = x0 * oc[j] + x1 * os[j];
                            Op[c][x][2 * j + 1] = x1 * oc[j] - x0 * os[j];
                            const float nc = oc[j] * sc[j] - os[j] * ss[j];
                            os[j] = os[j] * sc[j] + oc[j] * ss[j];
                            oc[j] = nc;
                        }
                }
            }
            if (a.out_bf16)
                store_rows(c, Op[c], sVst + (c & 1) * F::VTILE, gq[c % 2]);
            else
                store_out(c, Op[c]);
        }
    });

    // The state after the last token of the sequence: gamma^(tokens) R_in + the local end state.
    if (last && a.state_out) {
        const float gT = gpow(lg, (float)seg_n);
        float* out = a.state_out + (long long)pair * DK * adv;
#pragma unroll
        for (int x = 0; x < F::NKB; ++x) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[(long long)(x * 16 + g4 + e) * adv + dv0 + w * 16 + n16] = gT * Rin[x][e] + R[x][e];
        }
    }
    chain_finish(a, 64, DK * 64, s_word);
}

}  // namespace ret
