// Retention score normalizations ("Hybrid Architectures: RetNet and the Three Computation Paradigms", section
// 8.5; RetNet paper summary, "Retention Score Normalization"): scores scaled by 1/sqrt(d_k), the decay matrix's
// rows divided by the square root of their sums, and each row of scores divided by max(|row sum|, 1). Each is a
// factor per output row, so the normalized output is the plain one times
//     c_p / den_p,   c_p = [1/sqrt(d_k)] [1/sqrt(sum_{i=0}^{p} gamma^i)],   den_p = max(|c_p q'_p . z_p|, 1)
// for the row of absolute position p, where z_p = gamma z_{p-1} + k'_p is the decayed sum of the rotated keys:
// the row sum of the scores is q'_p . z_p. The rows refer to the whole sequence from its first token, so a call
// that resumes at pos0 carries z in and out beside the state.
//
// Chunkwise: the sequence is cut into segments of kNormSegTokens tokens; norm_zseg_kernel sums each segment's
// keys from zero, the segment scan (segment_scan_kernel, d_v = 1) turns those into the sum entering every
// segment, norm_rows_kernel runs the scan through its segment and writes each row's factor, and
// norm_scale_kernel scales the output rows in place. A decode step: norm_step_kernel updates z and scales the
// step's output row.
//
// Lane layout: lane l of the one wave of a (segment, b*H + h) owns rotation pairs l and l + 64 (NPL pairs); per
// token it loads the pairs' q and k values (4 bytes each in bf16), rotates them by their exact factors (fp64
// angle reduced by pi/2, fp32 Taylor sine and cosine) and updates its part of z. Tokens move through a ring of
// RING blocks of TB tokens whose loads are issued RING blocks ahead (64 tokens in flight, or 32 where a token's
// values take twice the registers); the partial dot products of a ring's tokens meet in LDS, where lane t sums
// token t's row.
#include "chunk_bf16.h"

namespace ret {

namespace {

constexpr int TB = 16;    // tokens per load block

// c_p of a row at absolute position p (fp64: 1 - gamma^(p+1) loses every digit in fp32 for gamma near 1).
__device__ __forceinline__ double norm_c(int norm, int dk, double lng, long long p) {
    double c = 1.0;
    if (norm & 1) c = 1.0 / sqrt((double)dk);
    if (norm & 2) {
        const double s = lng == 0.0 ? (double)(p + 1) : expm1((double)(p + 1) * lng) / expm1(lng);
        c /= sqrt(s);
    }
    return c;
}
__device__ __forceinline__ float norm_factor(int norm, int dk, double lng, long long p, float qz) {
    const double c = norm_c(norm, dk, lng, p);
    double den = 1.0;
    if (norm & 4) {
        const double r = fabs(c * (double)qz);
        den = r > 1.0 ? r : 1.0;
    }
    return (float)(c / den);
}

// Two consecutive input values (one rotation pair) widened to fp32.
template <class E>
struct PairLoad;
template <>
struct PairLoad<BF16> {
    typedef uint32_t raw;
    static constexpr int bytes = 4;
    __device__ static __forceinline__ raw load(rsrc_t r, int voff, int soff) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    }
    __device__ static __forceinline__ void widen(raw x, float& a, float& b) {
        a = __uint_as_float(x << 16);
        b = __uint_as_float(x & 0xffff0000u);
    }
};
template <>
struct PairLoad<F32> {
    typedef uint32_t __attribute__((ext_vector_type(2))) raw;
    static constexpr int bytes = 8;
    __device__ static __forceinline__ raw load(rsrc_t r, int voff, int soff) {
        return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    }
    __device__ static __forceinline__ void widen(raw x, float& a, float& b) {
        a = __uint_as_float(x[0]);
        b = __uint_as_float(x[1]);
    }
};

// The scan of z through tokens [t0, t0 + n) of one (b, h), starting from z; with ROWS, each token's q'.z goes to
// LDS and, per 64 tokens, lane t turns token t's sum into the row factor f. Loads of tokens past n read zero
// (the resources end at the segment's last row) and those tokens are skipped.
template <class E, int NPL, bool ROWS>
__device__ __forceinline__ void norm_scan(const NormArgs& a, int b, int h, long long t0, int n, float (&z)[NPL][2],
                                          float (*sp)[65]) {
    typedef PairLoad<E> PL;
    // blocks in flight: 128 registers of raw loads per lane (q and k of 64 tokens x one bf16 pair)
    constexpr int RING = 4 / (NPL * PL::bytes / 4);
    constexpr int GT = RING * TB;  // tokens of one LDS reduction
    const int lane = threadIdx.x;
    const int npairs = a.dk / 2;
    const int rowb = a.H * a.dk * PL::bytes / 2;  // bytes between tokens
    const long long head0 = ((long long)b * a.N + t0) * a.H + h;
    const int rbytes = n > 0 ? (n - 1) * rowb + a.dk * PL::bytes / 2 : 0;
    const rsrc_t rk = bytes_rsrc((const char*)a.k + head0 * a.dk * PL::bytes / 2, rbytes);
    const rsrc_t rq = bytes_rsrc((const char*)a.q + head0 * a.dk * PL::bytes / 2, ROWS ? rbytes : 0);
    int voff[NPL];
    bool live[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int pi = lane + 64 * j;
        live[j] = pi < npairs;
        voff[j] = live[j] ? pi * PL::bytes : 0x40000000;  // idle lanes read past the range: zero
    }
    const float g = a.gamma[h];
    const int nblk = (n + TB - 1) / TB;
    typename PL::raw bk[RING][TB][NPL], bq[RING][TB][NPL];
    auto issue = [&](int blk, auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
#pragma unroll
        for (int i = 0; i < TB; ++i)
#pragma unroll
            for (int j = 0; j < NPL; ++j) {
                const int soff = (blk * TB + i) * rowb;
                bk[r][i][j] = PL::load(rk, voff[j], soff);
                if constexpr (ROWS) bq[r][i][j] = PL::load(rq, voff[j], soff);
            }
    };
    static_for<0, RING>([&](auto rc) __attribute__((always_inline)) { issue(decltype(rc)::value, rc); });
    for (int blk0 = 0; blk0 < nblk; blk0 += RING) {
        static_for<0, RING>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            const int blk = blk0 + r;
#pragma unroll
            for (int i = 0; i < TB; ++i) {
                const int t = blk * TB + i;
                float part = 0.f;
                if (t < n) {
                    const long long p = a.pos0 + t0 + t;
#pragma unroll
                    for (int j = 0; j < NPL; ++j) {
                        float k0, k1, q0 = 0.f, q1 = 0.f;
                        PL::widen(bk[r][i][j], k0, k1);
                        if constexpr (ROWS) PL::widen(bq[r][i][j], q0, q1);
                        if (a.rotate && live[j]) {
                            float c, s;
                            rot_cs(p, a.theta[lane + 64 * j], &c, &s);
                            const float k0r = k0 * c - k1 * s, k1r = k0 * s + k1 * c;
                            const float q0r = q0 * c - q1 * s, q1r = q0 * s + q1 * c;
                            k0 = k0r; k1 = k1r; q0 = q0r; q1 = q1r;
                        }
                        z[j][0] = g * z[j][0] + k0;
                        z[j][1] = g * z[j][1] + k1;
                        part += q0 * z[j][0] + q1 * z[j][1];
                    }
                }
                if constexpr (ROWS) sp[(r * TB + i)][lane] = part;
            }
            issue(blk + RING, rc);
        });
        if constexpr (ROWS) {
            __syncthreads();
            // lane t < GT: token blk0*TB + t
            float r = 0.f;
#pragma unroll 16
            for (int l = 0; l < 64; ++l) r += sp[lane][l];
            const int t = blk0 * TB + lane;
            if (lane < GT && t < n) {
                const long long p = a.pos0 + t0 + t;
                a.f[((long long)b * a.N + t0 + t) * a.H + h] = norm_factor(a.norm, a.dk, a.lng[h], p, r);
            }
            __syncthreads();
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the ring's last loads (past the segment) are done before the wave ends
}

template <class E, int NPL>
__global__ __launch_bounds__(64) void norm_zseg_kernel(NormArgs a) {
    const int seg = blockIdx.x, pair = blockIdx.y, b = pair / a.H, h = pair % a.H;
    const long long t0 = (long long)seg * a.seg_len;
    const int n = (int)min((long long)a.seg_len, (long long)a.N - t0);
    float z[NPL][2];
#pragma unroll
    for (int j = 0; j < NPL; ++j) z[j][0] = z[j][1] = 0.f;
    norm_scan<E, NPL, false>(a, b, h, t0, n, z, nullptr);
    // the local end sum of segment seg is slot seg + 1 (the segment scan adds the earlier ones)
    float* w = a.W + ((long long)pair * a.nseg + seg + 1) * a.dk;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int pi = threadIdx.x + 64 * j;
        if (pi < a.dk / 2) *reinterpret_cast<float2*>(w + 2 * pi) = make_float2(z[j][0], z[j][1]);
    }
}

template <class E, int NPL>
__global__ __launch_bounds__(64) void norm_rows_kernel(NormArgs a) {
    __shared__ float sp[64][65];
    const int seg = blockIdx.x, pair = blockIdx.y, b = pair / a.H, h = pair % a.H;
    const long long t0 = (long long)seg * a.seg_len;
    const int n = (int)min((long long)a.seg_len, (long long)a.N - t0);
    const float* w = a.W + ((long long)pair * a.nseg + seg) * a.dk;  // the sum entering the segment
    float z[NPL][2];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int pi = threadIdx.x + 64 * j;
        const float2 x = pi < a.dk / 2 ? *reinterpret_cast<const float2*>(w + 2 * pi) : make_float2(0.f, 0.f);
        z[j][0] = x.x;
        z[j][1] = x.y;
    }
    norm_scan<E, NPL, true>(a, b, h, t0, n, z, sp);
    if (seg == a.nseg - 1 && a.z_out) {
        float* zo = a.z_out + (long long)pair * a.dk;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const int pi = threadIdx.x + 64 * j;
            if (pi < a.dk / 2) *reinterpret_cast<float2*>(zo + 2 * pi) = make_float2(z[j][0], z[j][1]);
        }
    }
}

// o[row][:] *= f[row]: thread i scales values 8i .. 8i+7 (d_v is a multiple of 8).
__global__ __launch_bounds__(256) void norm_scale_kernel(NormArgs a) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long total = (long long)a.B * a.N * a.H * a.dv / 8;
    if (i >= total) return;
    const long long e = 8 * i;
    const float f = a.f[e / a.dv];
    float x[8];
    if (a.out_bf16) {
        uint4* p = reinterpret_cast<uint4*>((uint16_t*)a.o + e);
        unpack8_bf16(*p, x);
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] *= f;
        *p = pack8_bf16(x);
    } else {
        float4* p = reinterpret_cast<float4*>((float*)a.o + e);
        float4 u = p[0], v = p[1];
        p[0] = make_float4(u.x * f, u.y * f, u.z * f, u.w * f);
        p[1] = make_float4(v.x * f, v.y * f, v.z * f, v.w * f);
    }
}

// A decode step: z <- gamma z + k' (in place: each (b, h) reads its row of z before writing it), then the step's
// output row times its factor. Rotation factors from the host (one position for the call).
template <class E, int NPL>
__global__ __launch_bounds__(64) void norm_step_kernel(NormArgs a) {
    typedef typename E::st st;
    const int pair = blockIdx.x, h = pair % a.H, lane = threadIdx.x;
    const float g = a.gamma[h];
    const st* qp = (const st*)a.q + (long long)pair * a.dk;
    const st* kp = (const st*)a.k + (long long)pair * a.dk;
    const float* zi = a.z_in ? a.z_in + (long long)pair * a.dk : nullptr;
    float zr[NPL][2], part = 0.f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int pi = lane + 64 * j;
        zr[j][0] = zr[j][1] = 0.f;
        if (pi < a.dk / 2) {
            float q0, q1, k0, k1;
            if constexpr (sizeof(st) == 2) {
                const uint32_t uq = *reinterpret_cast<const uint32_t*>(qp + 2 * pi);
                const uint32_t uk = *reinterpret_cast<const uint32_t*>(kp + 2 * pi);
                q0 = __uint_as_float(uq << 16); q1 = __uint_as_float(uq & 0xffff0000u);
                k0 = __uint_as_float(uk << 16); k1 = __uint_as_float(uk & 0xffff0000u);
            } else {
                const float2 uq = *reinterpret_cast<const float2*>(qp + 2 * pi);
                const float2 uk = *reinterpret_cast<const float2*>(kp + 2 * pi);
                q0 = uq.x; q1 = uq.y; k0 = uk.x; k1 = uk.y;
            }
            if (a.rotate) {
                const float c = a.rc[pi], s = a.rs[pi];
                const float q0r = q0 * c - q1 * s, q1r = q0 * s + q1 * c;
                const float k0r = k0 * c - k1 * s, k1r = k0 * s + k1 * c;
                q0 = q0r; q1 = q1r; k0 = k0r; k1 = k1r;
            }
            float2 z0 = zi ? *reinterpret_cast<const float2*>(zi + 2 * pi) : make_float2(0.f, 0.f);
            zr[j][0] = g * z0.x + k0;
            zr[j][1] = g * z0.y + k1;
            part += q0 * zr[j][0] + q1 * zr[j][1];
        }
    }
#pragma unroll
    for (int m = 1; m < 64; m *= 2) part += __shfl_xor(part, m);
    const float f = norm_factor(a.norm, a.dk, a.lng[h], a.pos0, part);
    if (a.z_out) {
        float* zo = a.z_out + (long long)pair * a.dk;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const int pi = lane + 64 * j;
            if (pi < a.dk / 2) *reinterpret_cast<float2*>(zo + 2 * pi) = make_float2(zr[j][0], zr[j][1]);
        }
    }
    for (int c = 4 * lane; c < a.dv; c += 256) {
        const long long e = (long long)pair * a.dv + c;
        if (a.out_bf16) {
            uint2* p = reinterpret_cast<uint2*>((uint16_t*)a.o + e);
            const uint2 u = *p;
            const float x0 = __uint_as_float(u.x << 16) * f, x1 = __uint_as_float(u.x & 0xffff0000u) * f;
            const float x2 = __uint_as_float(u.y << 16) * f, x3 = __uint_as_float(u.y & 0xffff0000u) * f;
            *p = make_uint2(pack2_bf16(x0, x1), pack2_bf16(x2, x3));
        } else {
            float4* p = reinterpret_cast<float4*>((float*)a.o + e);
            const float4 x = *p;
            *p = make_float4(x.x * f, x.y * f, x.z * f, x.w * f);
        }
    }
}

template <class E, int NPL>
NormKernels norm_set() {
    return {norm_zseg_kernel<E, NPL>, norm_rows_kernel<E, NPL>, norm_scale_kernel, norm_step_kernel<E, NPL>};
}

}  // namespace

bool norm_kernels_get(bool bf16_in, int dk, NormKernels* out) {
    if (dk <= 0 || dk % 2 || dk > 2 * kMaxPairs) return false;
    if (dk <= 128) *out = bf16_in ? norm_set<BF16, 1>() : norm_set<F32, 1>();
    else *out = bf16_in ? norm_set<BF16, 2>() : norm_set<F32, 2>();
    return true;
}

}  // namespace ret
