// Device helpers for the gfx950 retention kernels: element traits, bf16 rounding, MFMA tile products,
// global->LDS staging with the position rotation, and the decay factors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ret {

constexpr int kThreads = 256;   // 4 wave64s per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kMaxHeads = 64;
constexpr int kMaxPairs = 128;  // rotation frequencies per head: d_k <= 256

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// s_waitcnt immediate that waits until at most n vector memory operations of the wave are outstanding (and
// for nothing else). Those complete in the order they were issued, so this waits for all but the n latest.
__host__ __device__ constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) & 3) << 14 | 7 << 4 | 15 << 8; }

// ---------------------------------------------------------------------------------------------------
// bf16 <-> fp32. Rounding to bf16 is round-to-nearest-even by the gfx950 packed conversion
// (v_cvt_pk_bf16_f32); NaN stays NaN.
// ---------------------------------------------------------------------------------------------------
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)(pack2_bf16(f, 0.f) & 0xffffu); }

// ---------------------------------------------------------------------------------------------------
// Element traits. `st` is the storage type in global memory and LDS. KD is the MFMA reduction depth of one
// 16x16 instruction; PAD pads LDS rows (16 bytes) so that the 16 rows one MFMA operand reads spread over
// the LDS banks.
// ---------------------------------------------------------------------------------------------------
struct BF16 {
    typedef uint16_t st;
    static constexpr int KD = 32;
    static constexpr int PAD = 8;
};
struct F32 {
    typedef float st;
    static constexpr int KD = 4;
    static constexpr int PAD = 4;
};

// 8 consecutive elements from global memory, widened to fp32.
__device__ __forceinline__ void load8(const uint16_t* p, float* f) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float* p, float* f) {
    float4 a = reinterpret_cast<const float4*>(p)[0];
    float4 b = reinterpret_cast<const float4*>(p)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// 8 consecutive fp32 values stored (rounded to the storage type) to LDS.
__device__ __forceinline__ void store8(uint16_t* p, const float* f) {
    uint4 u;
    u.x = pack2_bf16(f[0], f[1]);
    u.y = pack2_bf16(f[2], f[3]);
    u.z = pack2_bf16(f[4], f[5]);
    u.w = pack2_bf16(f[6], f[7]);
    *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float* f) {
    reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
}

// 4 consecutive fp32 values to LDS storage (8 bytes for bf16, 16 for fp32).
__device__ __forceinline__ void store4(uint16_t* p, f32x4_t v) {
    uint2 u;
    u.x = pack2_bf16(v[0], v[1]);
    u.y = pack2_bf16(v[2], v[3]);
    *reinterpret_cast<uint2*>(p) = u;
}
__device__ __forceinline__ void store4(float* p, f32x4_t v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void store_out(uint16_t* p, float f) { *p = f32_to_bf16(f); }
__device__ __forceinline__ void store_out(float* p, float f) { *p = f; }

// Packed bf16 rows: 8 values in one uint4 (element 2i in the low half of word i).
__device__ __forceinline__ uint4 pack8_bf16(const float* f) {
    return make_uint4(pack2_bf16(f[0], f[1]), pack2_bf16(f[2], f[3]), pack2_bf16(f[4], f[5]),
                      pack2_bf16(f[6], f[7]));
}
__device__ __forceinline__ void unpack8_bf16(uint4 u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ uint32_t word(const uint4& u, int i) { return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w; }

// Transpose of an 8x8 block of packed bf16 rows: column e of rows 0..7 into out[e].
__device__ __forceinline__ void transpose8_bf16(const uint4* rows, uint4* out) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t w[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t a = word(rows[2 * m], e / 2), b = word(rows[2 * m + 1], e / 2);
            w[m] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        out[e] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// ---------------------------------------------------------------------------------------------------
// 16x16 output tile of C += A * B^T with A [16][k] and B [16][k] in LDS (k contiguous, row pitch lda/ldb
// elements), over k in [0, klen), klen a multiple of KD. Accumulator layout (both MFMA kinds): lane l holds
// C[4*(l/16) + i][l % 16], i = 0..3. Operand lanes pair row/column l % 16 with a k-group chosen by l / 16;
// A and B use the same k-group map, so the sum covers every k exactly once.
// ---------------------------------------------------------------------------------------------------
__device__ __forceinline__ void mma_nt(f32x4_t& acc, const uint16_t* A, int lda, const uint16_t* B, int ldb,
                                       int klen, int lane) {
    const uint16_t* a = A + (lane & 15) * lda + 8 * (lane >> 4);
    const uint16_t* b = B + (lane & 15) * ldb + 8 * (lane >> 4);
    for (int k = 0; k < klen; k += 32) {
        uint4 ua = *reinterpret_cast<const uint4*>(a + k);
        uint4 ub = *reinterpret_cast<const uint4*>(b + k);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ua),
                                                      __builtin_bit_cast(bf16x8_t, ub), acc, 0, 0, 0);
    }
}
__device__ __forceinline__ void mma_nt(f32x4_t& acc, const float* A, int lda, const float* B, int ldb, int klen,
                                       int lane) {
    const float* a = A + (lane & 15) * lda + (lane >> 4);
    const float* b = B + (lane & 15) * ldb + (lane >> 4);
    for (int k = 0; k < klen; k += 4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[k], b[k], acc, 0, 0, 0);
}

// One MFMA operand fragment: rows 0..15 of a k-contiguous LDS matrix at k offset k0 (the same lane map as
// mma_nt), so that a fragment shared by several tiles is read from LDS once.
__device__ __forceinline__ bf16x8_t frag(const uint16_t* M, int ld, int k0, int lane) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(M + (lane & 15) * ld + k0 + 8 * (lane >> 4)));
}
__device__ __forceinline__ float frag(const float* M, int ld, int k0, int lane) {
    return M[(lane & 15) * ld + k0 + (lane >> 4)];
}
__device__ __forceinline__ void mfma(f32x4_t& acc, bf16x8_t a, bf16x8_t b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma(f32x4_t& acc, float a, float b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// ---------------------------------------------------------------------------------------------------
// Decay and rotation factors.
// ---------------------------------------------------------------------------------------------------
// gamma^e for e >= 0 from log2(gamma) (computed on the host in fp64), by the hardware base-2 exponential
// (the exponent is <= 0, so results lie in (0, 1]; a result below the fp32 normal range becomes 0). Never the
// global factorisation gamma^n * gamma^-m, which overflows for long sequences.
__device__ __forceinline__ float gpow(float log2g, float e) { return __builtin_amdgcn_exp2f(e * log2g); }

// cos/sin of the angle p*theta. The angle is formed in fp64 and reduced there by the nearest multiple of pi/2
// (quadrant k), leaving r in [-pi/4, pi/4]; sin r and cos r then come from their Taylor series in fp32
// (through r^9 and r^10: truncation error below 2e-9), and the quadrant picks signs and swaps.
__device__ __forceinline__ void rot_cs(long long p, double theta, float* c, float* s) {
    const double half_pi = 1.5707963267948966192313216916398;
    const double a = (double)p * theta;
    const double kq = rint(a * (1.0 / half_pi));
    const float r = (float)(a - kq * half_pi);
    const float r2 = r * r;
    // sin r = r (1 - r^2/3! (1 - r^2/(4*5) (1 - r^2/(6*7) (1 - r^2/(8*9)))))
    float sr = 1.0f - r2 * (1.0f / 72.0f);
    sr = 1.0f - r2 * (1.0f / 42.0f) * sr;
    sr = 1.0f - r2 * (1.0f / 20.0f) * sr;
    sr = r * (1.0f - r2 * (1.0f / 6.0f) * sr);
    // cos r = 1 - r^2/2! (1 - r^2/(3*4) (1 - r^2/(5*6) (1 - r^2/(7*8) (1 - r^2/(9*10)))))
    float cr = 1.0f - r2 * (1.0f / 90.0f);
    cr = 1.0f - r2 * (1.0f / 56.0f) * cr;
    cr = 1.0f - r2 * (1.0f / 30.0f) * cr;
    cr = 1.0f - r2 * (1.0f / 12.0f) * cr;
    cr = 1.0f - r2 * 0.5f * cr;
    const int q = (int)((long long)kq & 3);
    const float sv = (q & 1) ? cr : sr, cv = (q & 1) ? sr : cr;
    *s = (q & 2) ? -sv : sv;
    *c = ((q + 1) & 2) ? -cv : cv;
}

// ---------------------------------------------------------------------------------------------------
// Staging of a chunk tile. Work unit = 8 tokens x 8 dims: 8 row loads of 8 elements, optional rotation,
// then row-layout stores (8 contiguous) and/or column-layout stores (an 8x8 transpose in registers).
// Tokens at or beyond `L` are zero-filled.
// ---------------------------------------------------------------------------------------------------
struct Seq {
    int N, H;
    int b, h;
};

template <class T>
__device__ __forceinline__ const T* row_ptr(const T* x, const Seq& s, int d, long long t, int d0) {
    return x + (((long long)s.b * s.N + t) * s.H + s.h) * d + d0;
}

// Rotation state of one staging unit: factors for the current token and the one-token step per pair.
struct RotUnit {
    float c[4], s[4], dc[4], ds[4];
    __device__ __forceinline__ void init(const double* theta, int pair0, long long p) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            rot_cs(p, theta[pair0 + j], &c[j], &s[j]);
            rot_cs(1, theta[pair0 + j], &dc[j], &ds[j]);
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
    __device__ __forceinline__ void step() {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float nc = c[j] * dc[j] - s[j] * ds[j];
            s[j] = s[j] * dc[j] + c[j] * ds[j];
            c[j] = nc;
        }
    }
};

// Q and K slice [d0, d0+W) of tokens [t0, t0+CT): Q -> sQ (row), K -> sK (row) and sKc (column, each token
// scaled by zeta_t before rounding); which destinations exist is fixed at compile time. Rotation uses the
// global pair index (d0 + c) / 2. Within a unit the rotation of token r+1 is that of token r turned by the
// one-token step (angle addition), so each unit evaluates two accurate sin/cos per pair instead of eight; q
// and k share the factors. Loads are branch-free (rows past L re-read row L-1 and are zeroed by a select), so
// all eight rows of a unit are in flight together. On the bf16 path the eight K rows wait for the transpose
// packed (4 registers per row).
template <class E, int CT, int W, bool HAS_Q, bool HAS_KROW, bool HAS_KCOL>
__device__ __forceinline__ void stage_qk(const typename E::st* q, const typename E::st* k, const Seq& s, int dk,
                                         long long t0, int L, int d0, const double* theta, bool rotate,
                                         long long pos0, float log2g, typename E::st* sQ, int ldq,
                                         typename E::st* sK, int ldk, typename E::st* sKc, int ldkc, int tid) {
    constexpr int UT = CT / 8, UD = W / 8;
    constexpr bool kBF16 = sizeof(typename E::st) == 2;
    for (int u = tid; u < UT * UD; u += kThreads) {
        const int tb = u / UD, db = u % UD;
        const int rs = s.H * dk;  // elements between consecutive tokens
        const typename E::st* qb = HAS_Q ? row_ptr(q, s, dk, t0 + tb * 8, d0 + db * 8) : nullptr;
        const typename E::st* kb = row_ptr(k, s, dk, t0 + tb * 8, d0 + db * 8);
        float qv[HAS_Q ? 8 : 1][8], kv[8][8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int tr = min(tb * 8 + r, L - 1) - tb * 8;  // clamp: never read past the sequence
            if constexpr (HAS_Q) load8(qb + tr * rs, qv[r]);
            load8(kb + tr * rs, kv[r]);
        }
        RotUnit rot;
        if (rotate) rot.init(theta, (d0 + db * 8) / 2, pos0 + t0 + tb * 8);
        uint4 kc16[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const bool live = tb * 8 + r < L;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (HAS_Q) qv[r][e] = live ? qv[r][e] : 0.f;
                kv[r][e] = live ? kv[r][e] : 0.f;
            }
            if (rotate) {
                if constexpr (HAS_Q) rot.apply(qv[r]);
                rot.apply(kv[r]);
                rot.step();
            }
            if constexpr (HAS_Q) store8(sQ + (tb * 8 + r) * ldq + db * 8, qv[r]);
            if constexpr (HAS_KROW) store8(sK + (tb * 8 + r) * ldk + db * 8, kv[r]);
            if constexpr (HAS_KCOL) {
                const float z = live ? gpow(log2g, (float)(L - 1 - (tb * 8 + r))) : 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[r][e] *= z;
                if constexpr (kBF16) kc16[r] = pack8_bf16(kv[r]);
            }
        }
        if constexpr (HAS_KCOL) {
            if constexpr (kBF16) {
                uint4 cols[8];
                transpose8_bf16(kc16, cols);
#pragma unroll
                for (int e = 0; e < 8; ++e) *reinterpret_cast<uint4*>(sKc + (db * 8 + e) * ldkc + tb * 8) = cols[e];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float col[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r) col[r] = kv[r][e];
                    store8(sKc + (db * 8 + e) * ldkc + tb * 8, col);
                }
            }
        }
    }
}

// V columns [d0, d0+W) of tokens [t0, t0+CT) -> sVc (column layout). bf16 rows move as packed words. Loads
// are branch-free as in stage_qk.
template <class E, int CT, int W>
__device__ __forceinline__ void stage_v(const typename E::st* v, const Seq& s, int dv, long long t0, int L, int d0,
                                        typename E::st* sVc, int ldvc, int tid) {
    constexpr int UT = CT / 8, UD = W / 8;
    for (int u = tid; u < UT * UD; u += kThreads) {
        const int tb = u / UD, db = u % UD;
        const typename E::st* vb = row_ptr(v, s, dv, t0 + tb * 8, d0 + db * 8);
        const int rs = s.H * dv;
        if constexpr (sizeof(typename E::st) == 2) {
            uint4 rows[8], cols[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int tr = min(tb * 8 + r, L - 1) - tb * 8;
                rows[r] = *reinterpret_cast<const uint4*>(vb + tr * rs);
            }
#pragma unroll
            for (int r = 0; r < 8; ++r)
                if (tb * 8 + r >= L) rows[r] = make_uint4(0u, 0u, 0u, 0u);
            transpose8_bf16(rows, cols);
#pragma unroll
            for (int e = 0; e < 8; ++e) *reinterpret_cast<uint4*>(sVc + (db * 8 + e) * ldvc + tb * 8) = cols[e];
        } else {
            float vv[8][8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int tr = min(tb * 8 + r, L - 1) - tb * 8;
                load8(vb + tr * rs, vv[r]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float col[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) col[r] = (tb * 8 + r < L) ? vv[r][e] : 0.f;
                store8(sVc + (db * 8 + e) * ldvc + tb * 8, col);
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------------
// Pipelined staging. An item is 8 consecutive tokens x IW consecutive dims of one tensor, kept in registers
// as raw words between issue_item() (the eight row loads; rows past L re-read row L-1, never past the
// sequence) and a commit (zero rows past L, rotate / scale, write LDS). Kernels issue the loads of stage i+1
// before computing stage i, so memory latency overlaps the MFMA work. Items are sized so that every thread
// of the workgroup holds one Q+K item and one V item per stage; q and k of an item share rotation factors.
// ---------------------------------------------------------------------------------------------------
template <class E, int IW>
struct Item {
    static constexpr int WPR = IW * (int)sizeof(typename E::st) / 4;  // 32-bit words per row
    uint32_t w[8][WPR];
};

template <int N>
__device__ __forceinline__ void load_words(uint32_t* w, const void* p) {
    if constexpr (N == 1) {
        w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else if constexpr (N == 2) {
        uint2 x = *reinterpret_cast<const uint2*>(p);
        w[0] = x.x; w[1] = x.y;
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            uint4 x = reinterpret_cast<const uint4*>(p)[i / 4];
            w[i] = x.x; w[i + 1] = x.y; w[i + 2] = x.z; w[i + 3] = x.w;
        }
    }
}
template <int N>
__device__ __forceinline__ void store_words(void* p, const uint32_t* w) {
    if constexpr (N == 1) {
        *reinterpret_cast<uint32_t*>(p) = w[0];
    } else if constexpr (N == 2) {
        *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 4) reinterpret_cast<uint4*>(p)[i / 4] = make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]);
    }
}

template <class E, int IW>
__device__ __forceinline__ void issue_item(Item<E, IW>& it, const typename E::st* base, int rs, int rows_live) {
#pragma unroll
    for (int r = 0; r < 8; ++r) load_words<Item<E, IW>::WPR>(it.w[r], base + min(r, rows_live - 1) * rs);
}

// Row r of an item widened to fp32 (zero past rows_live).
template <class E, int IW>
__device__ __forceinline__ void item_row(const Item<E, IW>& it, int r, int rows_live, float* f) {
    const bool live = r < rows_live;
    if constexpr (sizeof(typename E::st) == 2) {
#pragma unroll
        for (int i = 0; i < IW / 2; ++i) {
            const uint32_t x = live ? it.w[r][i] : 0u;
            f[2 * i] = __uint_as_float(x << 16);
            f[2 * i + 1] = __uint_as_float(x & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < IW; ++i) f[i] = live ? __uint_as_float(it.w[r][i]) : 0.f;
    }
}

// IW fp32 values stored as one row segment (rounded to the storage type).
template <class E, int IW>
__device__ __forceinline__ void store_row(typename E::st* dst, const float* f) {
    if constexpr (sizeof(typename E::st) == 2) {
        uint32_t w[IW / 2];
#pragma unroll
        for (int i = 0; i < IW / 2; ++i) w[i] = pack2_bf16(f[2 * i], f[2 * i + 1]);
        store_words<IW / 2>(dst, w);
    } else {
        uint32_t w[IW];
#pragma unroll
        for (int i = 0; i < IW; ++i) w[i] = __float_as_uint(f[i]);
        store_words<IW>(dst, w);
    }
}

// Column e of 8 rows x[r][e] stored as 8 consecutive tokens (16 bytes bf16, 32 bytes fp32).
template <class E, int IW>
__device__ __forceinline__ void store_col(typename E::st* dst, const float (&x)[8][IW], int e) {
    if constexpr (sizeof(typename E::st) == 2) {
        uint32_t w[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) w[m] = pack2_bf16(x[2 * m][e], x[2 * m + 1][e]);
        store_words<4>(dst, w);
    } else {
        uint32_t w[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) w[r] = __float_as_uint(x[r][e]);
        store_words<8>(dst, w);
    }
}

// Rotation of NP pairs along 8 consecutive tokens: the factors of the first token are evaluated accurately;
// each next token's factors are the previous ones turned by the one-token step (angle addition). The step
// factors (cos theta_i, sin theta_i) are evaluated once per kernel by the caller.
template <int NP>
struct RotStep {
    float dc[NP], ds[NP];
    __device__ __forceinline__ void init(const double* theta, int pair0) {
#pragma unroll
        for (int j = 0; j < NP; ++j) rot_cs(1, theta[pair0 + j], &dc[j], &ds[j]);
    }
};
template <int NP>
struct Rot8 {
    float c[NP], s[NP];
    __device__ __forceinline__ void init(const double* theta, int pair0, long long p0) {
#pragma unroll
        for (int j = 0; j < NP; ++j) rot_cs(p0, theta[pair0 + j], &c[j], &s[j]);
    }
    __device__ __forceinline__ void apply(float* x) const {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const float a0 = x[2 * j], a1 = x[2 * j + 1];
            x[2 * j] = a0 * c[j] - a1 * s[j];
            x[2 * j + 1] = a0 * s[j] + a1 * c[j];
        }
    }
    __device__ __forceinline__ void step(const RotStep<NP>& st) {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const float nc = c[j] * st.dc[j] - s[j] * st.ds[j];
            s[j] = s[j] * st.dc[j] + c[j] * st.ds[j];
            c[j] = nc;
        }
    }
};

// Q and K items of the same 8 tokens x IW dims: Q -> sQ rows, K -> sK rows and sKc columns (token r scaled
// by zeta[r] before rounding). Destinations are chosen at compile time.
template <class E, int IW, bool HAS_Q, bool HAS_KROW>
__device__ __forceinline__ void commit_qk(const Item<E, IW>* qi, const Item<E, IW>& ki, int rows_live, bool rotate,
                                          const double* theta, int pair0, long long p0, const RotStep<IW / 2>& rs,
                                          const float* zeta, typename E::st* dq, int ldq, typename E::st* dkr,
                                          int ldk, typename E::st* dkc, int ldc) {
    Rot8<IW / 2> rot;
    if (rotate) rot.init(theta, pair0, p0);
    float kx[8][IW];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        float qx[IW];
        if constexpr (HAS_Q) item_row<E, IW>(*qi, r, rows_live, qx);
        item_row<E, IW>(ki, r, rows_live, kx[r]);
        if (rotate) {
            if constexpr (HAS_Q) rot.apply(qx);
            rot.apply(kx[r]);
            rot.step(rs);
        }
        if constexpr (HAS_Q) store_row<E, IW>(dq + r * ldq, qx);
        if constexpr (HAS_KROW) store_row<E, IW>(dkr + r * ldk, kx[r]);
#pragma unroll
        for (int e = 0; e < IW; ++e) kx[r][e] *= zeta[r];
    }
#pragma unroll
    for (int e = 0; e < IW; ++e) store_col<E, IW>(dkc + e * ldc, kx, e);
}

// zeta[r] = gamma^(zexp0 - r) for the 8 rows of an item (0 for rows at or past rows_live).
__device__ __forceinline__ void item_zeta(float* zeta, float log2g, int zexp0, int rows_live) {
#pragma unroll
    for (int r = 0; r < 8; ++r) zeta[r] = r < rows_live ? gpow(log2g, (float)(zexp0 - r)) : 0.f;
}

// V item -> sVc columns.
template <class E, int IW>
__device__ __forceinline__ void commit_vcol(const Item<E, IW>& vi, int rows_live, typename E::st* dvc, int ldc) {
    float x[8][IW];
#pragma unroll
    for (int r = 0; r < 8; ++r) item_row<E, IW>(vi, r, rows_live, x[r]);
#pragma unroll
    for (int e = 0; e < IW; ++e) store_col<E, IW>(dvc + e * ldc, x, e);
}

// Item width for a CT x W tile: about one item per thread (at least one rotation pair, at most 8 dims), and
// the number of items each thread handles.
template <int CT, int W>
struct ItemWidth {
    static constexpr int raw = CT * W / (8 * kThreads);
    static constexpr int value = raw <= 2 ? 2 : raw <= 4 ? 4 : 8;
    static constexpr int count = (CT / 8) * (W / value);
    static constexpr int per_thread = (count + kThreads - 1) / kThreads;
    static_assert(W % value == 0, "item width");
};

}  // namespace ret
