// bf16-input chunkwise kernels (gfx950). Same computation as the generic chunk kernels in kernels.h, with a
// staging scheme built on two gfx950 features:
//  * buffer loads/stores whose resource covers exactly the live rows of the current chunk: rows past the end
//    of the sequence read as zero and stores to them are dropped, so no clamps, selects or guards, and the
//    row offsets are scalar (one per pass) on top of one per-thread offset fixed for the whole kernel;
//  * LDS transpose reads (ds_read_b64_tr_b16), so K and V live in LDS row-major only and the products that
//    contract over tokens (K^T V and V^T P^T) read them transposed.
// Each thread moves 16-byte row segments (8 dims of one token). The rotation factors of a thread's segment
// follow its tokens across passes and chunks by angle addition and are re-evaluated exactly every 8 chunks.
#pragma once

#include "kernels.h"

namespace ret {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Word 3 of a gfx9 buffer resource for raw (stride 0, 32-bit data format) access: every dword is range
// checked against the record count, loads out of range return 0 and stores out of range are dropped.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t bytes_rsrc(const void* base, int nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, kRawBufferWord3);
}
__device__ __forceinline__ u32x4_t buf_load16(rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// The same with the non-temporal hint, for rows a kernel reads once.
__device__ __forceinline__ u32x4_t buf_load16_nt(rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCachePolicyNT));
}
__device__ __forceinline__ void buf_store16(rsrc_t r, int voff, int soff, u32x4_t x) {
    __builtin_amdgcn_raw_buffer_store_b128(x, r, voff, soff, 0);
}

// Operand fragments in the permuted reduction order used by the fused kernel: within each 32-wide reduction
// step, lane group g (= lane / 16) holds indices 4g..4g+3 and 16+4g..16+4g+3. An MFMA sums over the reduction
// index, so any order shared by both operands gives the same product; this one matches the accumulator
// layout of a 16x16 tile (lane group g holds rows 4g..4g+3), so accumulators of two vertically adjacent
// tiles form an operand without leaving their lanes.
// Row-major X[m][k] (pitch ld): lane l receives X[l%16][k0 + 4g + i] and X[l%16][k0 + 16 + 4g + i].
__device__ __forceinline__ bf16x8_t frag_p(const uint16_t* X, int ld, int k0, int lane) {
    const uint16_t* p = X + (lane & 15) * ld + k0 + 4 * (lane >> 4);
    const uint2 lo = *reinterpret_cast<const uint2*>(p), hi = *reinterpret_cast<const uint2*>(p + 16);
    return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
}
// Transposed, from row-major X[k][n]: lane l receives X[k0 + 4g + i][n0 + l%16] and X[k0 + 16 + 4g + i][n0 + l%16].
// `tro` is trp_lane_offset(ld, lane).
__device__ __forceinline__ int trp_lane_offset(int ld, int lane) {
    return (4 * (lane >> 4) + ((lane >> 2) & 3)) * ld + 4 * (lane & 3);
}
__device__ __forceinline__ bf16x8_t frag_trp(const uint16_t* X, int ld, int k0, int n0, int tro) {
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
    uint16_t* p = const_cast<uint16_t*>(X) + k0 * ld + n0 + tro;
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p);
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p + 16 * ld));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// LDS tile of W bf16 columns laid out for both read patterns of the products. With 64 banks of 4 bytes the
// LDS serves a 64-lane 8-byte read as two halves of 32 lanes, and each half should touch all 64 banks once:
//  * row fragments (frag_ps): 16 consecutive rows x 2 adjacent 8-byte units;
//  * transposed fragments (frag_trps): 8 consecutive rows x 4 adjacent units.
// A row pitch of W + 16 columns (8 mod 16 words past a multiple of 64 banks) serves the second; swapping the two
// 8-column halves of every 16 columns in rows 8..15 of each 16 (c ^ 8) then also serves the first. The swap
// keeps 16-byte staging stores whole and does not interact with column offsets that are multiples of 16, so a
// lane's part of a fragment address is one value per tile and the rest are constants.
template <int W>
struct Swz {
    static constexpr int LD = W + 16;
    // element offset of column c (a multiple of 4) of row r
    __device__ static __forceinline__ int off(int r, int c) { return r * LD + (c ^ (((r >> 3) & 1) << 3)); }
    // lane part of frag_ps / frag_trps addresses
    __device__ static __forceinline__ int lane_p(int lane) { return off(lane & 15, 4 * (lane >> 4)); }
    __device__ static __forceinline__ int lane_trp(int lane) {
        return off(4 * (lane >> 4) + ((lane >> 2) & 3), 4 * (lane & 3));
    }
};
// frag_p on a Swz tile: rows r0 + l%16 (r0 a multiple of 16), reduction columns k0 + 4g.. and k0 + 16 + 4g..
// (k0 a multiple of 32). `lo_` is Swz<W>::lane_p(lane).
template <int W>
__device__ __forceinline__ bf16x8_t frag_ps(const uint16_t* X, int r0, int k0, int lo_) {
    const uint16_t* p = X + r0 * Swz<W>::LD + k0 + lo_;
    const uint2 lo = *reinterpret_cast<const uint2*>(p), hi = *reinterpret_cast<const uint2*>(p + 16);
    return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
}
// frag_trp on a Swz tile X[k][n]: lane l receives X[k0 + 4g + i][n0 + l%16] and X[k0 + 16 + 4g + i][n0 + l%16]
// (k0 a multiple of 32, n0 of 16). `lo_` is Swz<W>::lane_trp(lane).
template <int W>
__device__ __forceinline__ bf16x8_t frag_trps(const uint16_t* X, int k0, int n0, int lo_) {
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
    uint16_t* p = const_cast<uint16_t*>(X) + k0 * Swz<W>::LD + n0 + lo_;
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p);
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p + 16 * Swz<W>::LD));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Two accumulator tiles (rows 0..15 and 16..31 of a 32-row block) as one operand in the permuted order.
__device__ __forceinline__ bf16x8_t acc_pair(f32x4_t a, f32x4_t b) {
    return __builtin_bit_cast(bf16x8_t, make_uint4(pack2_bf16(a[0], a[1]), pack2_bf16(a[2], a[3]),
                                                   pack2_bf16(b[0], b[1]), pack2_bf16(b[2], b[3])));
}

// Rows of a T x W bf16 tile moved as 16-byte segments by NT threads: SPR segments per row, RP rows per pass of
// the workgroup, NP passes. Thread t owns segment t % SPR of rows t / SPR + p * RP.
template <int T, int W, int NT = kThreads>
struct RowTile {
    static constexpr int SPR = W / 8;
    static constexpr int RP = NT / SPR;
    static constexpr int NP = (T + RP - 1) / RP;
    static constexpr bool PARTIAL = T % RP != 0;
    static_assert(W % 8 == 0 && NT % SPR == 0, "row tile");
    __device__ static __forceinline__ bool live(int row0, int p) { return !PARTIAL || row0 + p * RP < T; }
};

// Rotation factors of the four pairs of one 16-byte segment.
struct Rot4 {
    float c[4], s[4];
    __device__ __forceinline__ void eval(long long p, const double* theta, int pair0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) rot_cs(p, theta[pair0 + j], &c[j], &s[j]);
    }
    // this <- this turned by st (angle addition)
    __device__ __forceinline__ void turn(const Rot4& st) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float nc = c[j] * st.c[j] - s[j] * st.s[j];
            s[j] = s[j] * st.c[j] + c[j] * st.s[j];
            c[j] = nc;
        }
    }
    __device__ __forceinline__ void apply(float* x) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float a0 = x[2 * j], a1 = x[2 * j + 1];
            x[2 * j] = a0 * c[j] - a1 * s[j];
            x[2 * j + 1] = a0 * s[j] + a1 * c[j];
        }
    }
};

__device__ __forceinline__ void unpack8(u32x4_t u, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(u[i] << 16);
        f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ u32x4_t pack8(const float* f) {
    return u32x4_t{pack2_bf16(f[0], f[1]), pack2_bf16(f[2], f[3]), pack2_bf16(f[4], f[5]), pack2_bf16(f[6], f[7])};
}
__device__ __forceinline__ void lds_store16(uint16_t* p, u32x4_t x) { *reinterpret_cast<u32x4_t*>(p) = x; }

// Per-thread rotation state of the Q/K segments of one d_k slice: the factors of the thread's row in the
// current pass (cur), the step between passes (RP tokens) and the step from the last pass of a chunk to the
// first of the next (C - (NP - 1) RP tokens; the same step unless the tile is partial). MODE 1: the chunks of a
// reversed run staged in memory order, each C rows before the one before it (a step of -C - (NP - 1) RP); MODE
// 2: the rows of a reversed run taken in the run's order, every step negated.
template <int C, int RP, int NP, int MODE = 0>
struct SliceRot {
    Rot4 cur, pass;
    Rot4 wrap;  // used only for partial tiles and reversed runs staged in memory order
    static constexpr bool SAME = MODE != 1 && C == NP * RP;
    __device__ __forceinline__ void init_steps(const double* theta, int pair0) {
        pass.eval(MODE == 2 ? -RP : RP, theta, pair0);
        if constexpr (!SAME)
            wrap.eval(MODE == 0 ? C - (NP - 1) * RP : MODE == 1 ? -(C + (NP - 1) * RP) : -(C - (NP - 1) * RP), theta,
                      pair0);
    }
    __device__ __forceinline__ void next_chunk() {
        if constexpr (SAME) cur.turn(pass);
        else cur.turn(wrap);
    }
};


// ---------------------------------------------------------------------------------------------------
// Segment chain. With nseg > 1 segments per sequence, the state entering segment s is
//   R_in(s) = sum_{j<s} gamma^((s-1-j) T) A_j + gamma^(s T) state_in,   T = tokens per segment,
// where A_j is segment j's end state from a zero start (its aggregate; the first segment's includes the
// decayed state_in, which then needs no term of its own). The workgroups of a unit (one d_v
// tile of one (b, h)) take their segments as tickets from the unit's counter, so every predecessor of a
// segment has started before it waits. Segments form groups of 8: a
// segment adds up the aggregates of the earlier segments of its group and the inclusive prefix I = R_in(g0)
// that enters the group, which the last segment of the previous group publishes (it computes its own R_in
// the same way). Every R_in is thus a sum in a fixed order, independent of timing, over at most 8 slots.
// Published states are written and read at device scope (sc1) and a slot's flag is raised only after the
// slot's stores completed (the ordering argument is below chain_wait); a wait that sees no progress for the
// call's limit (default ~0.17 s) gives up, sets the sticky error word and takes NaN for the entering state, so
// the outputs that depend on it are NaN instead of silently wrong. The unit's last workgroup past the look-back
// returns its counters and flags to zero.
// ---------------------------------------------------------------------------------------------------
constexpr int kOutAux = 0;                        // output stores: default policy (nt and sc1 measured no faster)
constexpr int kChainGroup = 8;                    // segments per look-back group
constexpr int kChainAux = 16;                     // buffer cache policy: sc1 (device-scope coherent)

// Waits until flags[lo .. lo+n) are all nonzero (n <= 64; lane i watches flag lo + i). False if it gave up: after
// `spin` ticks of the 100 MHz s_memrealtime clock in which no further flag rose (each flag that rises restarts
// the limit), or at once when spin < 0 (the host's way to exercise this path without a real stall).
//
// Ordering. A publisher stores its slot with device-scope (sc1) buffer stores, waits for them to complete
// (s_waitcnt vmcnt(0): on gfx9 a store is counted until the device-coherent level has acknowledged it), and only
// then stores the flag, itself a device-scope store. A waiter reads the flag with a device-scope load, and issues
// its slot loads only after the flag's value has come back (the ballot and the branch depend on it). Those slot
// loads are device-scope too: they are not served from the waiter's L1 or its XCD's L2, which may hold stale lines
// of the reused workspace, but from the device-coherent level, where the slot's stores had completed before the
// flag was written. So a waiter that sees the flag sees the slot. The same holds for the prefix slot and its flag
// value 2. (Release/acquire atomics would give the same guarantee through a write-back and an invalidation of
// the whole L2 per publication; these scoped accesses touch only the lines involved.)
__device__ __forceinline__ bool chain_wait(const int* flags, int lo, int n, int* error, long long spin) {
    const int lane = threadIdx.x & 63;
    if (spin < 0) {
        __hip_atomic_store(error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    int seen = 0;
    for (;;) {
        const int f = lane < n ? __hip_atomic_load(flags + lo + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1;
        const unsigned long long missing = __builtin_amdgcn_ballot_w64(f == 0);
        if (missing == 0) return true;
        const int up = 64 - __builtin_popcountll(missing);  // flags up (and idle lanes)
        const unsigned long long now = __builtin_amdgcn_s_memrealtime();
        if (up > seen) {  // progress: the limit counts from here
            seen = up;
            t0 = now;
        } else if (now - t0 > (unsigned long long)spin) {
            __hip_atomic_store(error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(4);
    }
}

// A pointer the caller knows to be wave-uniform, moved to scalar registers (the compiler cannot always prove
// it after divergent regions, and a buffer resource built from vector registers costs a loop per access).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
    const unsigned long long u = reinterpret_cast<unsigned long long>(p);
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u), hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
    return reinterpret_cast<T*>(((unsigned long long)hi << 32) | lo);
}

// One state slot: DK x (16 * NT / 64) floats in the thread order of the R tiles (tile x of thread t at
// (x*NT + t)*16 bytes).
template <int NKB, int NT>
__device__ __forceinline__ void slot_store(float* slot, const f32x4_t* R, int tid) {
    const rsrc_t r = bytes_rsrc(uniform_ptr(slot), NKB * NT * 16);
#pragma unroll
    for (int x = 0; x < NKB; ++x)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, R[x]), r, tid * 16, x * NT * 16, kChainAux);
}
template <int NKB, int NT>
__device__ __forceinline__ void slot_load(const float* slot, f32x4_t* v, int tid) {
    const rsrc_t r = bytes_rsrc(uniform_ptr(slot), NKB * NT * 16);
#pragma unroll
    for (int x = 0; x < NKB; ++x)
        v[x] = __builtin_bit_cast(f32x4_t,
                                  __builtin_amdgcn_raw_buffer_load_b128(r, tid * 16, x * NT * 16, kChainAux));
}

// The transpose of a square state slot (DK = DVT = 16 NW NDW) of another run into this thread's tiles:
// R[x NDW + j][e] is the slot's element (c, r) with r = 16x + g4 + e and c = 16(w NDW + j) + n16, which slot_store
// put in tile (c / 16) NDW + x % NDW of thread (x / NDW) 64 + (c % 16) / 4 * 16 + r % 16, component c % 4.
template <int NKB, int NDW, int NT>
__device__ __forceinline__ void slot_load_transposed(const float* slot, f32x4_t* R, int w, int g4, int n16) {
    const rsrc_t r = bytes_rsrc(uniform_ptr(slot), NKB * NDW * NT * 16);
#pragma unroll
    for (int x = 0; x < NKB; ++x)
#pragma unroll
        for (int j = 0; j < NDW; ++j) {
            const int c = 16 * (w * NDW + j) + n16;
            const int xs = (c / 16) * NDW + x % NDW;
            const int ts = (x / NDW) * 64 + (n16 / 4) * 16 + g4;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                R[x * NDW + j][e] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(r, ((xs * NT + ts + e) * 4 + n16 % 4) * 4, 0, 0));
        }
}

// The unit (one d_v tile of one (b, h)) of this workgroup, from the launch index. Workgroups are dispatched to
// the 8 XCDs in turn (launch index mod 8); when the grid divides evenly, the d_v tiles of one (b, h) get launch
// indices of one residue, so they run on one XCD and its L2 serves the q and k rows they all stage.
__device__ __forceinline__ int unit_of_block(int ntiles, int units) {
    const int pairs = units / ntiles;
    int unit_i;
    if (ntiles > 1 && gridDim.x % (8u * ntiles) == 0) {
        const int xcd = blockIdx.x % 8, q8 = blockIdx.x / 8;
        unit_i = ((q8 / ntiles * 8 + xcd) % pairs) * ntiles + q8 % ntiles;
    } else {
        unit_i = blockIdx.x % (unsigned)units;
    }
    return __builtin_amdgcn_readfirstlane(unit_i);
}

// The unit and segment of a workgroup of a grid of units x segments workgroups, segment-major. Workgroups go to
// the 8 XCDs in turn (launch index mod 8); when a segment's units divide evenly, the d_v tiles of one (b, h)
// get launch indices of one residue, so they run on one XCD and its L2 serves the q' and k' rows they all load.
__device__ __forceinline__ void unit_seg_of_block(int ntiles, int units, int* unit, int* seg) {
    const int bid = blockIdx.x, s = bid / units, r = bid % units;
    int u = r;
    if (ntiles > 1 && units % (8 * ntiles) == 0) {
        const int xcd = r % 8, q8 = r / 8;
        u = ((q8 / ntiles) * 8 + xcd) * ntiles + q8 % ntiles;
    }
    *unit = __builtin_amdgcn_readfirstlane(u);
    *seg = __builtin_amdgcn_readfirstlane(s);
}

// Chain storage of one unit (chained runs).
struct Chain {
    int* ctr;      // [2]: next segment ticket, workgroups past the look-back
    int* flags;    // [nseg]: nonzero once the segment's aggregate (or, for a group's last segment, the prefix
                   // leaving the group) is published
    float* agg;    // [nseg][slot]: aggregates
    float* inc;    // [nseg][slot]: prefixes leaving a group (published by its last segment)
    int* error;    // sticky error word of the header
    int slot;      // floats per state slot
    long long spin;  // wait limit (chain_wait)
};
__device__ __forceinline__ Chain chain_of(void* ws, int units, int nseg, int unit, int slot_floats,
                                          long long spin = 0) {
    const ChainLayout lay = chain_layout(units, nseg, slot_floats);
    char* base = reinterpret_cast<char*>(ws);
    Chain ch;
    ch.ctr = reinterpret_cast<int*>(base + lay.ctr_off) + 2 * unit;
    ch.flags = reinterpret_cast<int*>(base + lay.flags_off) + (size_t)unit * nseg;
    ch.agg = reinterpret_cast<float*>(base + lay.agg_off) + (size_t)unit * nseg * slot_floats;
    ch.inc = reinterpret_cast<float*>(base + lay.inc_off) + (size_t)unit * nseg * slot_floats;
    ch.error = &reinterpret_cast<ChainHeader*>(ws)->error;
    ch.slot = slot_floats;
    ch.spin = spin;
    return ch;
}

// The unit's next segment: a ticket from the unit's counter, broadcast through the shared word `bc`, so the
// workgroups that own a unit's earlier segments have all started.
__device__ __forceinline__ int chain_ticket(const Chain& ch, int& bc) {
    if (threadIdx.x == 0) bc = __hip_atomic_fetch_add(ch.ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int seg = __builtin_amdgcn_readfirstlane(bc);
    __syncthreads();
    return seg;
}


// Publishes segment seg's aggregate R (not for a group's last segment, whose flag announces the prefix).
// `then` may issue NTHEN vector memory operations per thread (loads the caller wants in flight early): they go
// out after the slot stores, and the wait before the flag covers the stores only. The flag store itself is
// not waited for here; the workgroup's count (chain_enter or chain_finish) waits for it first.
template <int NKB, int NT, int NTHEN, class Then>
__device__ __forceinline__ void chain_publish(const Chain& ch, int seg, const f32x4_t* R, Then&& then) {
    slot_store<NKB, NT>(ch.agg + (size_t)seg * ch.slot, R, threadIdx.x);
    __asm__ volatile("" ::: "memory");  // `then` stays behind the stores
    then();
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(NTHEN));
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(ch.flags + seg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <int NKB, int NT>
__device__ __forceinline__ void chain_publish(const Chain& ch, int seg, const f32x4_t* R) {
    chain_publish<NKB, NT, 0>(ch, seg, R, [] {});
}

// R_in of segment seg: the sum over the group's earlier segments j of gamma^((seg-1-j)T) A_j, plus
// gamma^((seg-g0)T) times the prefix entering the group (published by the previous group's last segment).
// If the wait gives up, R_in is NaN (and so is the prefix a group's last segment publishes from it).
// One poll covers every flag; slots are read in batches and added in a fixed order, so results do not depend
// on timing. A group's last segment (not the sequence's) then publishes gamma^T R_in + A_seg, A_seg = Rown.
// With COUNT, the workgroup then counts itself past the look-back and the unit's last one resets the unit's
// counters and flags (its other workgroups have read them all by then); without, chain_finish does that at
// the end of the kernel. `bc` is a shared broadcast word.
template <int NKB, int NT, bool COUNT>
__device__ __forceinline__ void chain_enter(const Chain& ch, int seg, int nseg, float gT, const f32x4_t* Rown,
                                            f32x4_t* Rin, int& bc) {
    const int tid = threadIdx.x;
    const int g0 = seg / kChainGroup * kChainGroup;              // first segment of this segment's group
    const bool boundary = seg % kChainGroup == kChainGroup - 1;  // publishes the prefix for the next group
    const bool last = seg == nseg - 1;
#pragma unroll
    for (int x = 0; x < NKB; ++x) Rin[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (seg > 0) {
        const int lo = g0 > 0 ? g0 - 1 : g0;
        // (wave-uniform: the wait's result is a ballot)
        const bool ok =
            __builtin_amdgcn_readfirstlane((int)chain_wait(ch.flags, lo, seg - lo, ch.error, ch.spin)) != 0;
        if (!ok) {
            const float nan = __builtin_nanf("");
#pragma unroll
            for (int x = 0; x < NKB; ++x) Rin[x] = f32x4_t{nan, nan, nan, nan};
        }
        constexpr int LB = NKB >= 16 ? 1 : NKB >= 8 ? 2 : 4;
        float dec = 1.f;
        for (int j0 = seg - 1; ok && j0 >= g0; j0 -= LB) {
            f32x4_t v[LB][NKB];
#pragma unroll
            for (int i = 0; i < LB; ++i)
                if (j0 - i >= g0) slot_load<NKB, NT>(ch.agg + (size_t)(j0 - i) * ch.slot, v[i], tid);
#pragma unroll
            for (int i = 0; i < LB; ++i)
                if (j0 - i >= g0) {
#pragma unroll
                    for (int x = 0; x < NKB; ++x) Rin[x] += dec * v[i][x];
                    dec *= gT;
                }
        }
        if (g0 > 0 && ok) {
            f32x4_t v[NKB];
            slot_load<NKB, NT>(ch.inc + (size_t)(g0 - 1) * ch.slot, v, tid);
#pragma unroll
            for (int x = 0; x < NKB; ++x) Rin[x] += dec * v[x];
        }
    }
    if (!last && boundary) {  // the prefix leaving the group: R_in of the next segment
        f32x4_t I[NKB];
#pragma unroll
        for (int x = 0; x < NKB; ++x) I[x] = gT * Rin[x] + Rown[x];
        slot_store<NKB, NT>(ch.inc + (size_t)seg * ch.slot, I, tid);
        __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    if (tid == 0 && !last && boundary) __hip_atomic_store(ch.flags + seg, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if constexpr (COUNT) {
        if (tid == 0) {
            __builtin_amdgcn_s_waitcnt(0);  // this workgroup's flag stores land before it counts
            bc = __hip_atomic_fetch_add(ch.ctr + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(bc) == nseg - 1) {
            for (int i = tid; i < nseg; i += (int)blockDim.x)
                __hip_atomic_store(ch.flags + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (tid == 0) {
                __hip_atomic_store(ch.ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(ch.ctr + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// At the end of the kernel: the workgroup counts itself finished, and the unit's last one resets the unit's
// counters and flags (the others are finished, so past every read of them). Counting only here keeps the
// counter's round trip off the path to the outputs where loads are in flight at the look-back: a vector
// atomic's result also waits for every load the wave issued before it. The unit's storage is located afresh from the workspace, so nothing stays live across
// the kernel for it. `bc` is a shared broadcast word.
__device__ __forceinline__ void chain_finish(const FwdArgs& a, int dvt, int slot_floats, int& bc) {
    const int ntiles = __builtin_amdgcn_readfirstlane(a.dv / dvt);
    const int units = __builtin_amdgcn_readfirstlane(a.B * a.H * ntiles);
    const int nseg = __builtin_amdgcn_readfirstlane(a.nseg);
    const Chain ch = chain_of(a.ws, units, nseg, unit_of_block(ntiles, units), slot_floats);
    const int tid = threadIdx.x;
    __syncthreads();
    if (tid == 0) {
        __builtin_amdgcn_s_waitcnt(0);  // this workgroup's flag stores land before it counts
        bc = __hip_atomic_fetch_add(ch.ctr + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(bc) == nseg - 1) {
        for (int i = tid; i < nseg; i += (int)blockDim.x)
            __hip_atomic_store(ch.flags + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0) {
            __hip_atomic_store(ch.ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ch.ctr + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------------------------------------------
// chunk_fused (bf16): one workgroup per (segment, d_v tile, b*H + h). Wave w owns NDW d_v blocks of 16 columns of
// every output and state tile. With several segments the workgroup first runs the local pass over its segment
// (R = sum over its chunks of gamma^(decay to the segment's end) (K (.) zeta)^T V, from zero, or from state_in for
// the first segment; split launches store it for the scan instead), publishes the end
// state and joins the segment chain for its entering state. The full pass then runs from that state: per
// chunk and d_k slice S^T = K Q^T (all lower-triangle tiles, kept in registers), the cross term
// O^T += R^T Q^T with R^T taken from the state accumulators and the state update; then
// O^T = xi (.) O^T + V^T P^T with P = mask (.) S straight from the S^T accumulators, stored to the output.
// ---------------------------------------------------------------------------------------------------
template <int DK, int C, int DVT, bool PRE, int NT, int NDW>
struct FullB {
    static constexpr int NW = NT / 64;  // waves; wave w owns d_v blocks w*NDW .. w*NDW + NDW - 1 of 16 columns
    static constexpr int KS = DK < 64 ? DK : 64;
    static constexpr int NSL = DK / KS;
    // q/k slices, V and the local pass's K are Swz tiles of KS, DVT and DK columns.
    static constexpr int NB = C / 16, NDV = DVT / 16, NKB = DK / 16, XB = KS / 16;
    static constexpr int NS = Tri<NB>::count;
    typedef RowTile<C, KS, NT> TQ;
    typedef RowTile<C, DVT, NT> TV;
    typedef RowTile<C, DK, NT> TK;  // local pass: whole d_k
    static constexpr int SQ = C * Swz<KS>::LD, SV = C * Swz<DVT>::LD;
    // One stage buffer: sQ, sK and (rotating in staging) sKz = K (.) zeta; with pre-rotated operands zeta goes
    // on the smaller V tile instead (sVz beside sV).
    static constexpr int STAGE = (PRE ? 2 : 3) * SQ;
    static constexpr int VBUF = (PRE ? 2 : 1) * SV;
    // With one d_k slice a chunk's V is read while the next chunk's is staged: two V buffers. With several,
    // V is read only in the first slice's products, a barrier ahead of the next chunk's staging: one.
    static constexpr int NVB = NSL == 1 ? 2 : 1;
    // Large d_k: each wave computes only its share of the S^T tiles and P goes through LDS, instead of every
    // wave computing all tiles (which costs NB(NB+1)/2 * d_k/32 MFMAs per wave per chunk).
    static constexpr bool SHARED_P = DK >= 128;
    static constexpr int NS_W = (NS + NW - 1) / NW;
    static constexpr int LDP = C + 8, SP = SHARED_P ? C * LDP : 0;
    static constexpr int FULL_BYTES = (2 * STAGE + NVB * VBUF + SP) * 2;
    static constexpr int LOCAL_BYTES = (C * Swz<DK>::LD + C * Swz<DVT>::LD) * 2;  // local pass: sKz [C][DK] and sV [C][DVT]
    static constexpr int LDS_BYTES = FULL_BYTES > LOCAL_BYTES ? FULL_BYTES : LOCAL_BYTES;
    // two workgroups per CU when the LDS allows and the registers of d_k = 256 are not needed
    static constexpr int OCC = LDS_BYTES <= 80 * 1024 && DK * NDW <= 128 ? 2 : 1;
    static_assert(NDV == NW * NDW, "NDW d_v blocks per wave");
    static_assert(C == 32 || C == 64, "chunk tile of 32 or 64 tokens");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(KS % 32 == 0, "tiling");
};

// REV: the run goes over the reversed sequence in place (token n of the run is row N-1-n of q, k, v and o; whole
// chunks only, N a multiple of C): the gradients' retentions over later tokens. Rows are rotated (q, k without
// PRE; v with a.vrot) by the rotation at their own positions in memory. GR (with PRE): the gradients' rotations
// of v rows (a.vrot) and of the outputs (a.orot) are compiled in.
template <int DK, int C, int DVT, bool PRE, int NT, int NDW, bool REV = false, bool GR = false>
__global__ __launch_bounds__(NT, (FullB<DK, C, DVT, PRE, NT, NDW>::OCC)) void chunk_fused_bf16(FwdArgs a) {
    typedef FullB<DK, C, DVT, PRE, NT, NDW> F;
    constexpr int NR = F::NKB * NDW;  // state tiles of a wave: R[x * NDW + j] = rows 16x.., d_v block w * NDW + j
    typedef typename F::TQ TQ;
    typedef typename F::TV TV;
    typedef typename F::TK TK;
    __shared__ __attribute__((aligned(16))) uint16_t smem[F::LDS_BYTES / 2];
    // Broadcast word (ticket, finish count): the first word of the staging region, which no thread writes
    // before a barrier that follows every read of it.
    int& s_word = *reinterpret_cast<int*>(smem);
    // Full pass: stage buffers (sQ, sK, sKz) alternate by stage, sV buffers by chunk.
    uint16_t* const stage_lds = smem;
    uint16_t* const v_lds = smem + 2 * F::STAGE;
    uint16_t* const sP = v_lds + F::NVB * F::VBUF;  // shared P (large d_k only)

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g4 = 4 * (lane >> 4), n16 = lane & 15;
    const int ntiles = __builtin_amdgcn_readfirstlane(a.dv / DVT);
    const int units = __builtin_amdgcn_readfirstlane(a.B * a.H * ntiles);
    // split 1: the local pass alone of every segment but the last, its state stored to the segment's slot;
    // split 2: the full pass alone of every segment, from the state in its slot (a scan of the local passes' states
    // in between); split 0: one launch, the segments chained.
    const int split = __builtin_amdgcn_readfirstlane(a.split);
    const bool chained = a.nseg > 1 && split == 0;
    // The unit comes from the launch index; with several segments the segment is the unit's next ticket.
    int unit, seg;
    if (split) {  // segment-major grids of units x segments
        unit_seg_of_block(ntiles, units, &unit, &seg);
    } else {
        unit = unit_of_block(ntiles, units);
        seg = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / (unsigned)units));
    }
    Chain ch{};
    if (chained) {
        ch = chain_of(a.ws, units, a.nseg, unit, DK * DVT, a.chain_spin);
        seg = chain_ticket(ch, s_word);
    }
    // Scalar arguments re-read as wave-uniform values: they are live across the divergent ticket branch.
    const int aN = __builtin_amdgcn_readfirstlane(a.N);
    const int aH = __builtin_amdgcn_readfirstlane(a.H), adk = __builtin_amdgcn_readfirstlane(a.dk);
    const int adv = __builtin_amdgcn_readfirstlane(a.dv), anseg = __builtin_amdgcn_readfirstlane(a.nseg);
    const int aseg_len = __builtin_amdgcn_readfirstlane(a.seg_len);
    const int pair = unit / ntiles;
    const int b = pair / aH, h = pair % aH;
    const int dv0 = (unit % ntiles) * DVT;
    const float lg = a.log2g[h];
    const long long seg_t0 = (long long)seg * aseg_len;
    const int seg_n = (int)(min((long long)aN, seg_t0 + aseg_len) - seg_t0);  // tokens in this segment
    const int nchunks = (seg_n + C - 1) / C;
    const int rsk = aH * adk, rsv = aH * adv;  // elements between consecutive tokens
    // token 0 of this (b, h), in head rows; the first row in memory of chunk c: token seg_t0 + c C of the run, or,
    // over the reversed sequence, row N - seg_t0 - (c + 1) C, whose C rows are the chunk's tokens in reverse order
    const long long hrow = (long long)b * aN * aH + h;
    auto crow = [&](int c) __attribute__((always_inline)) {
        return REV ? (long long)aN - seg_t0 - (long long)(c + 1) * C : seg_t0 + (long long)c * C;
    };
    // the chunk's row (and LDS row) of memory row r of its rows
    auto lrow = [&](int r) __attribute__((always_inline)) { return REV ? C - 1 - r : r; };
    // q and k, or their rotated copies (PRE: staging copies rows instead of rotating them)
    const uint16_t* qh = (const uint16_t*)(PRE ? a.qr : a.q) + hrow * adk;
    const uint16_t* kh = (const uint16_t*)(PRE ? a.kr : a.k) + hrow * adk;
    const uint16_t* vh = (const uint16_t*)a.v + hrow * adv + dv0;
    const int osz = a.out_bf16 ? 2 : 4;
    char* oh = (char*)a.o + (hrow * adv + dv0) * osz;
    const int vrow = tid / TV::SPR, vseg = tid % TV::SPR;
    const int voff = (vrow * rsv + vseg * 8) * 2;
    typedef Swz<F::KS> ZQ;
    typedef Swz<DVT> ZV;
    typedef Swz<DK> ZK;
    const int lq_p = ZQ::lane_p(lane), lq_t = ZQ::lane_trp(lane), lv_t = ZV::lane_trp(lane);
    // State_in enters through the first segment: its local pass starts from it, so its published end state
    // carries state_in into every later R_in, and its full pass starts from it again.
    auto load_state_in = [&](f32x4_t* R) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < F::NKB; ++x)
#pragma unroll
            for (int j = 0; j < NDW; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    R[x * NDW + j][e] = a.state_in[((long long)pair * DK + x * 16 + g4 + e) * adv + dv0 +
                                                   (w * NDW + j) * 16 + n16];
    };

    // slot s of this unit (split launches): DK x DVT floats in the thread order of slot_store
    auto split_slot = [&](int s) __attribute__((always_inline)) {
        return a.ws + ((size_t)unit * anseg + s) * (size_t)(DK * DVT);
    };
    f32x4_t R[NR];
#pragma unroll
    for (int x = 0; x < NR; ++x) R[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (split == 2) {
        // (GR with a square state: a.ws_t, the transposes of another run's states, e.g. the gradients' dk' from the
        // dv retention's)
        if constexpr (PRE && GR && DK == DVT) {
            if (a.ws_t)
                slot_load_transposed<F::NKB, NDW, NT>(a.ws_t + ((size_t)unit * anseg + seg) * (size_t)(DK * DVT), R,
                                                      w, g4, n16);
            else
                slot_load<NR, NT>(split_slot(seg), R, tid);
        } else {
            slot_load<NR, NT>(split_slot(seg), R, tid);
        }
    } else if (seg == 0 && a.state_in) {
        load_state_in(R);
        if (split == 1) {  // the scan starts from state_in, in slot 0; the local pass itself from zero
            slot_store<NR, NT>(split_slot(0), R, tid);
#pragma unroll
            for (int x = 0; x < NR; ++x) R[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    } else if (split == 1 && seg == 0) {
        slot_store<NR, NT>(split_slot(0), R, tid);  // zero
    }

    const bool last = seg == anseg - 1;
    const bool boundary = seg % kChainGroup == kChainGroup - 1;  // a group's last segment publishes a prefix

    // ---- local pass over the segment (chained or split runs, all segments but the last) ----
    if ((chained || split == 1) && !last) {
        uint16_t* lK = smem;
        uint16_t* lV = smem + C * ZK::LD;
        const int lk_t = ZK::lane_trp(lane);
        const int krow = tid / TK::SPR, kseg = tid % TK::SPR;
        const int koff = (krow * rsk + kseg * 8) * 2;
        // The chunks are taken last first: step s adds chunk n-1-s (n chunks) scaled by gamma^(sC), its decay to
        // the segment's end, so the state is never rescaled and the sum is the same (measured 62 -> 56-57 us per
        // call for the local passes of long-sequence). Two register buffers: the loads of step s+2 go out as soon
        // as step s is staged.
        u32x4_t lk[2][TK::NP], lv[2][TV::NP];
        auto lissue = [&](int st, auto parc) __attribute__((always_inline)) {
            constexpr int par = decltype(parc)::value;
            const long long tc = crow(nchunks - 1 - st);
            const rsrc_t rk = bytes_rsrc(kh + tc * rsk, ((C - 1) * rsk + DK) * 2);
            const rsrc_t rv = bytes_rsrc(vh + tc * rsv, ((C - 1) * rsv + DVT) * 2);
#pragma unroll
            for (int p = 0; p < TK::NP; ++p) lk[par][p] = buf_load16(rk, koff, p * TK::RP * rsk * 2);
#pragma unroll
            for (int p = 0; p < TV::NP; ++p) lv[par][p] = buf_load16(rv, voff, p * TV::RP * rsv * 2);
        };
        lissue(0, std::integral_constant<int, 0>{});
        if (nchunks > 1) lissue(1, std::integral_constant<int, 1>{});
        float zl[TK::NP], zlv[TV::NP];
#pragma unroll
        for (int p = 0; p < TK::NP; ++p) zl[p] = gpow(lg, (float)(C - 1 - lrow(krow + p * TK::RP)));
#pragma unroll
        for (int p = 0; p < TV::NP; ++p) zlv[p] = gpow(lg, (float)(C - 1 - lrow(vrow + p * TV::RP)));
        // rotation factors of the thread's k rows (without PRE), or v rows (PRE with a.vrot): the step between
        // passes, and from the last pass of a chunk to the first of the chunk taken next, the one before it in the
        // run (C rows earlier in memory, or later over the reversed sequence; identity factors without rotation:
        // theta all zero)
        constexpr int LRP = PRE ? TV::RP : TK::RP, LNP = PRE ? TV::NP : TK::NP;
        const int lpair0 = PRE ? (dv0 + vseg * 8) / 2 : kseg * 4;
        const int lrow0 = PRE ? vrow : krow;
        constexpr bool VR = PRE && GR;  // (v rotation compiled in)
        const bool lrot_on = !PRE || (VR && a.vrot);
        Rot4 lrcur, lrpass, lrback;
        if (lrot_on) {
            lrpass.eval(LRP, a.theta, lpair0);
            lrback.eval(REV ? C - (LNP - 1) * LRP : -(C + (LNP - 1) * LRP), a.theta, lpair0);
        }
        // Step st of the local pass: chunk c = n-1-st (segments before the last hold whole chunks only).
        auto lchunk = [&](int st, auto parc) __attribute__((always_inline)) {
            constexpr int par = decltype(parc)::value;
            const int c = nchunks - 1 - st;
            const float gs = gpow(lg, (float)(st * C));  // decay of the chunk's end to the segment's end
            if (st > 0) __syncthreads();
            if (lrot_on && (st & 7) == 0) lrcur.eval(a.pos0 + crow(c) + lrow0, a.theta, lpair0);
            if constexpr (PRE) {  // K' as staged; zeta on V (turned by the rotation first with a.vrot)
#pragma unroll
                for (int p = 0; p < TK::NP; ++p)
                    if (TK::live(krow, p)) lds_store16(lK + ZK::off(lrow(krow + p * TK::RP), kseg * 8), lk[par][p]);
#pragma unroll
                for (int p = 0; p < TV::NP; ++p)
                    if (TV::live(vrow, p)) {
                        float vf[8];
                        unpack8(lv[par][p], vf);
                        if (VR && a.vrot) {
                            lrcur.apply(vf);
                            if (p + 1 < TV::NP) lrcur.turn(lrpass);
                        }
                        const float z = zlv[p] * gs;
#pragma unroll
                        for (int e = 0; e < 8; ++e) vf[e] *= z;
                        lds_store16(lV + ZV::off(lrow(vrow + p * TV::RP), vseg * 8), pack8(vf));
                    }
                if (VR && a.vrot) lrcur.turn(lrback);
            } else {
#pragma unroll
                for (int p = 0; p < TK::NP; ++p)
                    if (TK::live(krow, p)) {
                        float kf[8];
                        unpack8(lk[par][p], kf);
                        lrcur.apply(kf);
                        if (p + 1 < TK::NP) lrcur.turn(lrpass);
                        const float z = zl[p] * gs;
#pragma unroll
                        for (int e = 0; e < 8; ++e) kf[e] *= z;
                        lds_store16(lK + ZK::off(lrow(krow + p * TK::RP), kseg * 8), pack8(kf));
                    }
                lrcur.turn(lrback);
#pragma unroll
                for (int p = 0; p < TV::NP; ++p)
                    if (TV::live(vrow, p)) lds_store16(lV + ZV::off(lrow(vrow + p * TV::RP), vseg * 8), lv[par][p]);
            }
            if (st + 2 < nchunks) lissue(st + 2, parc);
            __syncthreads();
#pragma unroll
            for (int f = 0; f < C / 32; ++f) {
                bf16x8_t fb[NDW];
#pragma unroll
                for (int j = 0; j < NDW; ++j) fb[j] = frag_trps<DVT>(lV, 32 * f, (w * NDW + j) * 16, lv_t);
#pragma unroll
                for (int x = 0; x < F::NKB; ++x) {
                    const bf16x8_t ka = frag_trps<DK>(lK, 32 * f, x * 16, lk_t);
#pragma unroll
                    for (int j = 0; j < NDW; ++j) mfma(R[x * NDW + j], ka, fb[j]);
                }
            }
        };
        // (chained runs: the first segment's local pass starts from state_in, decayed here to the segment's end)
        if (chained && seg == 0 && a.state_in) {
            const float gL = gpow(lg, (float)(nchunks * C));
#pragma unroll
            for (int x = 0; x < NR; ++x) R[x] *= gL;
        }
        for (int st = 0; st < nchunks; st += 2) {
            lchunk(st, std::integral_constant<int, 0>{});
            if (st + 1 < nchunks) lchunk(st + 1, std::integral_constant<int, 1>{});
        }
        __syncthreads();  // the local tiles are dead before the full pass reuses the LDS
        if (split == 1) {  // the segment's state, for the scan
            slot_store<NR, NT>(split_slot(seg + 1), R, tid);
            return;
        }
        // Publish the aggregate for the later segments of the group (nothing else in flight). The first segment
        // starts its full pass from state_in again: it reloads it into R behind the slot stores and before its
        // flag rises, since state_out may be the same buffer, and the last segment writes it only after every
        // earlier segment's flag (segment 0 is never a group's last segment, so it always publishes here).
        if (!boundary) {
            if (seg == 0 && a.state_in)
                chain_publish<NR, NT, 0>(ch, seg, R, [&] { load_state_in(R); });
            else
                chain_publish<NR, NT>(ch, seg, R);
        }
    }

    // ---- full pass: staging ----
    const int qrow = tid / TQ::SPR, qseg = tid % TQ::SPR;
    const int qoff = (qrow * rsk + qseg * 8) * 2;
    // Two register buffers of staged loads: stage i+2's loads go out as soon as stage i is staged. Stage
    // parity is the chunk's with one d_k slice, the slice's with an even number of slices.
    constexpr int NBUF = 2;
    static_assert(F::NSL == 1 || F::NSL % 2 == 0, "stage parity");
    u32x4_t bq[NBUF][TQ::NP], bk[NBUF][TQ::NP], bv[NBUF][TV::NP];
    auto issue = [&](int i, auto parc) __attribute__((always_inline)) {
        constexpr int par = decltype(parc)::value;
        const int c = i / F::NSL, sl = i % F::NSL;
        const int L = min(C, seg_n - c * C);
        const long long tc = crow(c);
        const rsrc_t rq = bytes_rsrc(qh + tc * rsk + sl * F::KS, ((L - 1) * rsk + F::KS) * 2);
        const rsrc_t rk = bytes_rsrc(kh + tc * rsk + sl * F::KS, ((L - 1) * rsk + F::KS) * 2);
#pragma unroll
        for (int p = 0; p < TQ::NP; ++p) {
            bq[par][p] = buf_load16(rq, qoff, p * TQ::RP * rsk * 2);
            bk[par][p] = buf_load16(rk, qoff, p * TQ::RP * rsk * 2);
        }
        if (sl == 0) {
            const rsrc_t rv = bytes_rsrc(vh + tc * rsv, ((L - 1) * rsv + DVT) * 2);
#pragma unroll
            for (int p = 0; p < TV::NP; ++p) bv[par][p] = buf_load16(rv, voff, p * TV::RP * rsv * 2);
        }
    };
    const int nst = nchunks * F::NSL;
    if (nst > 0) issue(0, std::integral_constant<int, 0>{});
    if constexpr (NBUF == 2)
        if (nst > 1) issue(1, std::integral_constant<int, 1>{});

    // ---- entering state: state_in for the first segment (already back in R), else R_in from the chain ----
    if (chained) {
        f32x4_t Rin[NR];
        chain_enter<NR, NT, true>(ch, seg, anseg, gpow(lg, (float)aseg_len), R, Rin, s_word);
        if (seg > 0 || !a.state_in) {  // (segment 0's R_in is zero)
#pragma unroll
            for (int x = 0; x < NR; ++x) R[x] = Rin[x];
        }
    }

    // Chunk-independent decay factors: the mask gamma^(j-l) for S^T tiles Delta = jb - lb blocks below the
    // diagonal (rows l, columns j of the lane), xi_j = gamma^(j+1) of each O^T tile (column j) and zeta of
    // each staged row of a full chunk.
    float Dm[F::NB][4], Xi[F::NB], zfull[TQ::NP];
#pragma unroll
    for (int d = 0; d < F::NB; ++d)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int jl = 16 * d + n16 - g4 - e;  // j - l
            Dm[d][e] = jl >= 0 ? gpow(lg, (float)jl) : 0.f;
        }
#pragma unroll
    for (int x = 0; x < F::NB; ++x) Xi[x] = gpow(lg, (float)(x * 16 + n16 + 1));
    // Shared-P layout: S^T tile slot x of wave w is lower-triangle tile w + 4x (slots past the last tile repeat
    // it; their results are never stored), with its mask factors.
    int Sjb[F::NS_W], Slb[F::NS_W];
    f32x4_t DmS[F::NS_W];
    if constexpr (F::SHARED_P) {
#pragma unroll
        for (int x = 0; x < F::NS_W; ++x) {
            tri_tile<F::NB>(min(w + F::NW * x, F::NS - 1), Sjb[x], Slb[x]);
#pragma unroll
            for (int e = 0; e < 4; ++e) DmS[x][e] = Dm[Sjb[x] - Slb[x]][e];
        }
    }
#pragma unroll
    for (int p = 0; p < TQ::NP; ++p) zfull[p] = gpow(lg, (float)(C - 1 - lrow(qrow + p * TQ::RP)));
    float zvfull[TV::NP];  // zeta of the staged V rows of a full chunk (pre-rotated operands)
#pragma unroll
    for (int p = 0; p < TV::NP; ++p) zvfull[p] = gpow(lg, (float)(C - 1 - lrow(vrow + p * TV::RP)));
    const float gC = gpow(lg, (float)C);
    // Without rotation theta is all zero and every factor is exactly (1, 0).
    SliceRot<C, TQ::RP, TQ::NP, REV ? 1 : 0> rot[F::NSL];
    if constexpr (!PRE) {
#pragma unroll
        for (int sl = 0; sl < F::NSL; ++sl) rot[sl].init_steps(a.theta, (sl * F::KS + qseg * 8) / 2);
    }
    // PRE with a.vrot: the factors of the thread's v rows, as those of q and k without PRE
    SliceRot<C, TV::RP, TV::NP, REV ? 1 : 0> vrot;
    const int vpair0 = (dv0 + vseg * 8) / 2;
    constexpr bool VRF = PRE && GR;  // (v rotation compiled in)
    if constexpr (VRF)
        if (a.vrot) vrot.init_steps(a.theta, vpair0);

    auto commit = [&](int i, auto parc, auto slc) __attribute__((always_inline)) {
        constexpr int par = decltype(parc)::value, sl = decltype(slc)::value;
        const int c = i / F::NSL;
        const int L = min(C, seg_n - c * C);
        uint16_t* sQ = stage_lds + (i & 1) * F::STAGE;
        uint16_t* sK = sQ + F::SQ;
        uint16_t* sV = v_lds + (F::NVB == 2 ? (c & 1) * F::VBUF : 0);
        if constexpr (PRE) {
            // rows as staged; V also scaled by zeta into sVz
#pragma unroll
            for (int p = 0; p < TQ::NP; ++p)
                if (TQ::live(qrow, p)) {
                    lds_store16(sQ + ZQ::off(lrow(qrow + p * TQ::RP), qseg * 8), bq[par][p]);
                    lds_store16(sK + ZQ::off(lrow(qrow + p * TQ::RP), qseg * 8), bk[par][p]);
                }
            if constexpr (sl == 0) {
                uint16_t* sVz = sV + F::SV;
                if (VRF && a.vrot && (c & 7) == 0) vrot.cur.eval(a.pos0 + crow(c) + vrow, a.theta, vpair0);
#pragma unroll
                for (int p = 0; p < TV::NP; ++p) {
                    const int r = lrow(vrow + p * TV::RP);
                    if (TV::live(vrow, p)) {
                        const float z = L == C ? zvfull[p] : (r < L ? gpow(lg, (float)(L - 1 - r)) : 0.f);
                        float vf[8];
                        unpack8(bv[par][p], vf);
                        if (VRF && a.vrot) {
                            vrot.cur.apply(vf);
                            if (p + 1 < TV::NP) vrot.cur.turn(vrot.pass);
                            lds_store16(sV + ZV::off(r, vseg * 8), pack8(vf));
                        } else {
                            lds_store16(sV + ZV::off(r, vseg * 8), bv[par][p]);
                        }
#pragma unroll
                        for (int e = 0; e < 8; ++e) vf[e] *= z;
                        lds_store16(sVz + ZV::off(r, vseg * 8), pack8(vf));
                    }
                }
                if (VRF && a.vrot) vrot.next_chunk();
            }
        } else {
            uint16_t* sKz = sK + F::SQ;
            if ((c & 7) == 0)  // exact factors every 8 chunks; angle addition in between
                rot[sl].cur.eval(a.pos0 + crow(c) + qrow, a.theta, (sl * F::KS + qseg * 8) / 2);
#pragma unroll
            for (int p = 0; p < TQ::NP; ++p) {
                const int r = lrow(qrow + p * TQ::RP);
                if (TQ::live(qrow, p)) {
                    float qf[8], kf[8];
                    unpack8(bq[par][p], qf);
                    unpack8(bk[par][p], kf);
                    rot[sl].cur.apply(qf);
                    rot[sl].cur.apply(kf);
                    if (p + 1 < TQ::NP) rot[sl].cur.turn(rot[sl].pass);
                    lds_store16(sQ + ZQ::off(r, qseg * 8), pack8(qf));
                    lds_store16(sK + ZQ::off(r, qseg * 8), pack8(kf));
                    const float z = L == C ? zfull[p] : (r < L ? gpow(lg, (float)(L - 1 - r)) : 0.f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) kf[e] *= z;
                    lds_store16(sKz + ZQ::off(r, qseg * 8), pack8(kf));
                }
            }
            rot[sl].next_chunk();
            if constexpr (sl == 0) {
#pragma unroll
                for (int p = 0; p < TV::NP; ++p)
                    if (TV::live(vrow, p)) lds_store16(sV + ZV::off(lrow(vrow + p * TV::RP), vseg * 8), bv[par][p]);
            }
        }
    };

    // Output stores straight from the O^T accumulators: lane (g, n16) of tile (x, j) holds 4 consecutive d_v of
    // query x*16 + n16 in d_v block w * NDW + j (REV: memory row (NB-1-x)*16 + 15 - n16 of the chunk's rows). Rows
    // past the sequence fall outside the buffer range and are dropped.
    const int o_voff = ((REV ? 15 - n16 : n16) * rsv + w * NDW * 16 + g4) * osz;
    // a.orot (PRE only, for the gradients): every output row turned back by the transpose of the rotation at its
    // position. The lane's values of tile (x, j) are columns dv0 + (w NDW + j) 16 + g4 .. + 3 (two pairs) of run
    // row seg_t0 + c C + 16 x + n16, at position pos0 + that row (REV: pos0 + N - 1 - that row). The factors of a
    // chunk's first tile are evaluated exactly every 8 chunks and otherwise carried from the chunk before by angle
    // addition; those of the later tiles follow by steps of 16 rows.
    float oc[NDW][2], os[NDW][2], o16c[NDW][2], o16s[NDW][2], oCc[NDW][2], oCs[NDW][2];
    if constexpr (PRE && GR) {
        if (a.orot) {
#pragma unroll
            for (int j = 0; j < NDW; ++j)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const double th = a.theta[(dv0 + (w * NDW + j) * 16 + g4) / 2 + e];
                    rot_cs(REV ? -16 : 16, th, &o16c[j][e], &o16s[j][e]);
                    rot_cs(REV ? -C : C, th, &oCc[j][e], &oCs[j][e]);
                }
        }
    }
    auto out_rotate = [&](int c, f32x4_t* O) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NDW; ++j)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                if ((c & 7) == 0) {
                    const long long r = seg_t0 + (long long)c * C + n16;
                    rot_cs(a.pos0 + (REV ? (long long)aN - 1 - r : r), a.theta[(dv0 + (w * NDW + j) * 16 + g4) / 2 + e],
                           &oc[j][e], &os[j][e]);
                } else {
                    const float nc = oc[j][e] * oCc[j][e] - os[j][e] * oCs[j][e];
                    os[j][e] = os[j][e] * oCc[j][e] + oc[j][e] * oCs[j][e];
                    oc[j][e] = nc;
                }
                float cx = oc[j][e], sx = os[j][e];
#pragma unroll
                for (int x = 0; x < F::NB; ++x) {
                    const float x0 = O[x * NDW + j][2 * e], x1 = O[x * NDW + j][2 * e + 1];
                    O[x * NDW + j][2 * e] = x0 * cx + x1 * sx;
                    O[x * NDW + j][2 * e + 1] = x1 * cx - x0 * sx;
                    if (x + 1 < F::NB) {
                        const float nc = cx * o16c[j][e] - sx * o16s[j][e];
                        sx = sx * o16c[j][e] + cx * o16s[j][e];
                        cx = nc;
                    }
                }
            }
    };
    auto store_out = [&](int c, f32x4_t* O) __attribute__((always_inline)) {
        if constexpr (PRE && GR)
            if (a.orot) out_rotate(c, O);
        const int L = min(C, seg_n - c * C);
        const rsrc_t ro = bytes_rsrc(oh + crow(c) * rsv * osz, ((L - 1) * rsv + DVT) * osz);
        if (a.out_bf16) {
#pragma unroll
            for (int x = 0; x < F::NB; ++x)
#pragma unroll
                for (int j = 0; j < NDW; ++j)
                    __builtin_amdgcn_raw_buffer_store_b64(
                        __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(2))),
                                           make_uint2(pack2_bf16(O[x * NDW + j][0], O[x * NDW + j][1]),
                                                      pack2_bf16(O[x * NDW + j][2], O[x * NDW + j][3]))),
                        ro, o_voff, ((REV ? F::NB - 1 - x : x) * 16 * rsv + j * 16) * 2, kOutAux);
        } else {
#pragma unroll
            for (int x = 0; x < F::NB; ++x)
#pragma unroll
                for (int j = 0; j < NDW; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, O[x * NDW + j]), ro, o_voff,
                                                           ((REV ? F::NB - 1 - x : x) * 16 * rsv + j * 16) * 4,
                                                           kOutAux);
        }
    };

    // S^T tile (jb, lb), lb <= jb, in row-by-row lower-triangle order.
    auto tri = [](int jb, int lb) constexpr { return jb * (jb + 1) / 2 + lb; };
    constexpr int KF = C / 32;  // reduction steps over the tokens of a chunk

    // Products of stage i (chunk c, slice sl) from its stage buffer: S^T += K_s Q_s^T (all lower-triangle
    // tiles: every wave needs all of P), the cross term O^T += R_s^T Q_s^T with R^T taken from the state
    // accumulators (the previous chunk's state: this slice's update follows), and R_s <- gamma^L R_s +
    // (K_s (.) zeta)^T V.
    auto mma = [&](int i, auto slc, f32x4_t* S, f32x4_t* O, bf16x8_t* fv, bf16x8_t* fvz, float gL)
                   __attribute__((always_inline)) {
        constexpr int sl = decltype(slc)::value;
        const int c = i / F::NSL;
        const uint16_t* sQ = stage_lds + (i & 1) * F::STAGE;
        const uint16_t* sK = sQ + F::SQ;
        // state update operands: (K (.) zeta)^T V, or with pre-rotated operands K^T (V (.) zeta)
        const uint16_t* sKA = PRE ? sK : sK + F::SQ;
        const uint16_t* sV = v_lds + (F::NVB == 2 ? (c & 1) * F::VBUF : 0);
#pragma unroll
        for (int kk = 0; kk < F::KS; kk += 32) {
            bf16x8_t qf[F::NB], kf[F::NB];
#pragma unroll
            for (int x = 0; x < F::NB; ++x) {
                qf[x] = frag_ps<F::KS>(sQ, x * 16, kk, lq_p);
                if constexpr (!F::SHARED_P) kf[x] = frag_ps<F::KS>(sK, x * 16, kk, lq_p);
            }
            if constexpr (F::SHARED_P) {
#pragma unroll
                for (int x = 0; x < F::NS_W; ++x)
                    mfma(S[x], frag_ps<F::KS>(sK, Slb[x] * 16, kk, lq_p), frag_ps<F::KS>(sQ, Sjb[x] * 16, kk, lq_p));
            } else {
#pragma unroll
                for (int jb = 0; jb < F::NB; ++jb)
#pragma unroll
                    for (int lb = 0; lb <= jb; ++lb) mfma(S[tri(jb, lb)], kf[lb], qf[jb]);
            }
            const int rb = (sl * F::KS + kk) / 16;
#pragma unroll
            for (int j = 0; j < NDW; ++j) {
                const bf16x8_t ra = acc_pair(R[rb * NDW + j], R[(rb + 1) * NDW + j]);
#pragma unroll
                for (int x = 0; x < F::NB; ++x) mfma(O[x * NDW + j], ra, qf[x]);
            }
        }
        if constexpr (sl == 0) {
#pragma unroll
            for (int f = 0; f < KF; ++f)
#pragma unroll
                for (int j = 0; j < NDW; ++j) {
                    fv[f * NDW + j] = frag_trps<DVT>(sV, 32 * f, (w * NDW + j) * 16, lv_t);
                    if constexpr (PRE) fvz[f * NDW + j] = frag_trps<DVT>(sV + F::SV, 32 * f, (w * NDW + j) * 16, lv_t);
                }
        }
#pragma unroll
        for (int x = sl * F::XB * NDW; x < (sl + 1) * F::XB * NDW; ++x) R[x] *= gL;
#pragma unroll
        for (int f = 0; f < KF; ++f) {
#pragma unroll
            for (int x = sl * F::XB; x < (sl + 1) * F::XB; ++x) {
                const bf16x8_t ka = frag_trps<F::KS>(sKA, 32 * f, (x - sl * F::XB) * 16, lq_t);
#pragma unroll
                for (int j = 0; j < NDW; ++j) mfma(R[x * NDW + j], ka, PRE ? fvz[f * NDW + j] : fv[f * NDW + j]);
            }
        }
    };

    // Software pipeline over stages: stage i's products and stage i+1's staging (rotation, rounding, LDS
    // writes into the other buffers) run back to back with no barrier between them, so the vector work of
    // the staging issues while the matrix instructions execute; one barrier per stage.
    if constexpr (F::SHARED_P)  // scores above the diagonal are never written: zero for the P.V product
        for (int i = tid; i < F::SP; i += NT) sP[i] = 0;
    __syncthreads();  // every wave has read the broadcast word, which the first commit overwrites
    if (nst > 0) {
        commit(0, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
        if (NBUF < nst) issue(NBUF, std::integral_constant<int, 0>{});
    }
    __syncthreads();
    auto chunk = [&](int c, auto cparc) __attribute__((always_inline)) {
        constexpr int cpar = decltype(cparc)::value;
        const int L = min(C, seg_n - c * C);
        const float gL = L == C ? gC : gpow(lg, (float)L);
        constexpr int NSA = F::SHARED_P ? F::NS_W : F::NS;  // S^T accumulators of this wave
        f32x4_t S[NSA], O[F::NB * NDW];
#pragma unroll
        for (int x = 0; x < NSA; ++x) S[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int x = 0; x < F::NB * NDW; ++x) O[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // V^T operands of the wave's d_v blocks (A of the P.V product; B of the state update unless PRE), and
        // (V (.) zeta)^T: B of the state update with pre-rotated operands
        bf16x8_t fv[KF * NDW], fvz[KF * NDW];
        static_for<0, F::NSL>([&](auto slc) __attribute__((always_inline)) {
            constexpr int sl = decltype(slc)::value;
            constexpr int sln = (sl + 1) % F::NSL;  // slice of the next stage
            // register buffer of the next stage (stage parity is chunk parity when NBUF = 2: NSL = 1 then)
            constexpr int parn = F::NSL == 1 ? 1 - cpar : (sl + 1) & 1;
            const int i = c * F::NSL + sl;
            mma(i, slc, S, O, fv, fvz, gL);
            if (i + 1 < nst) {
                commit(i + 1, std::integral_constant<int, parn>{}, std::integral_constant<int, sln>{});
                if (i + 1 + NBUF < nst) issue(i + 1 + NBUF, std::integral_constant<int, parn>{});
            }
            if constexpr (sl == F::NSL - 1 && F::SHARED_P) {
                // P = mask (.) S^T of this wave's tiles into LDS (4 consecutive keys of one query per lane),
                // then O^T = xi (.) (R^T Q^T) + V^T P^T with P read back in the permuted key order.
#pragma unroll
                for (int x = 0; x < F::NS_W; ++x)
                    if (w + F::NW * x < F::NS) store4(sP + (Sjb[x] * 16 + n16) * F::LDP + Slb[x] * 16 + g4, S[x] * DmS[x]);
                __syncthreads();
#pragma unroll
                for (int x = 0; x < F::NB * NDW; ++x) O[x] *= Xi[x / NDW];
#pragma unroll
                for (int f = 0; f < KF; ++f) {
#pragma unroll
                    for (int x = 2 * f; x < F::NB; ++x) {
                        const bf16x8_t pf = frag_p(sP + x * 16 * F::LDP, F::LDP, 32 * f, lane);
#pragma unroll
                        for (int j = 0; j < NDW; ++j) mfma(O[x * NDW + j], fv[f * NDW + j], pf);
                    }
                }
                store_out(c, O);
            } else if constexpr (sl == F::NSL - 1) {
                // O^T = xi (.) (R^T Q^T) + V^T P^T, P = mask (.) S taken from the S^T accumulators as the B
                // operand (keys 32f.. of query block x are tiles lb = 2f and 2f + 1).
#pragma unroll
                for (int x = 0; x < F::NB * NDW; ++x) O[x] *= Xi[x / NDW];
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
                        const bf16x8_t pb = acc_pair(p0, p1);
#pragma unroll
                        for (int j = 0; j < NDW; ++j) mfma(O[x * NDW + j], fv[f * NDW + j], pb);
                    }
                }
                store_out(c, O);
            }
            __syncthreads();
        });
    };

    for (int c = 0; c < nchunks; c += 2) {
        chunk(c, std::integral_constant<int, 0>{});
        if (c + 1 < nchunks) chunk(c + 1, std::integral_constant<int, 1>{});
    }

    // The state after the last token of the sequence.
    if (last && a.state_out) {
        float* out = a.state_out + (long long)pair * DK * adv;
#pragma unroll
        for (int x = 0; x < F::NKB; ++x)
#pragma unroll
            for (int j = 0; j < NDW; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    out[(long long)(x * 16 + g4 + e) * adv + dv0 + (w * NDW + j) * 16 + n16] = R[x * NDW + j][e];
    }
}

// Chunks of 128 tokens run as 64-token sub-chunks: the chunkwise recurrence gives the same result for any
// chunk size (up to rounding), and 64-token tiles keep all of P in registers.
// Workgroups of 256 threads (4 waves, d_v tiles of 64), or d_v tiles of 128 where d_k is 256: one d_v tile's
// products are d_k-deep, so a wider tile shares the scores and the q/k staging among twice the columns. The
// wider tile is either 8 waves of 16 columns (two waves per SIMD hide each other's latencies) or 4 waves of
// NDW = 2 blocks of 16 columns (each Q', K' or P fragment read from LDS feeds two MFMAs).
// WITH_REV: the set also has the PRE kernel over the reversed sequence (fused_rev).
template <int DK, int C, int NT = (DK >= 256 ? 512 : 256), int NDW = 1, bool WITH_REV = false>
ChunkKernels chunk_entry_bf16() {
    constexpr int CI = C > 64 ? 64 : C, DVT = 16 * (NT / 64) * NDW;
    ChunkKernels k{};
    k.fused = chunk_fused_bf16<DK, CI, DVT, false, NT, NDW>;
    // (the sets with reversed instances serve the gradients: their PRE instances rotate outputs and v rows)
    k.fused_pre = chunk_fused_bf16<DK, CI, DVT, true, NT, NDW, false, WITH_REV>;
    if constexpr (WITH_REV) {
        k.fused_rev = chunk_fused_bf16<DK, CI, DVT, true, NT, NDW, true, true>;
        k.fused_rot_rev = chunk_fused_bf16<DK, CI, DVT, false, NT, NDW, true>;
        k.rev_step = CI;
    }
    k.dvt = DVT;
    k.threads = NT;
    k.fused_orot = WITH_REV;
    // d_v tiles of 128 run one workgroup per CU: one workgroup per CU in total measured fastest (fewer, longer
    // segments); 256-thread ones with 16-column waves two per CU, with two rounds of them.
    k.target_wgs = NT * NDW >= 512 ? 256 : 1024;
    return k;
}

}  // namespace ret
