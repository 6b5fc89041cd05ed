// Reordering and rotation of [B, N, H, d] tensors for the gradients of chunkwise retention.
//
// The gradients of L = sum(dO (.) O), O the retention output from a zero state, are themselves retentions
// (they follow from the parallel form, "Hybrid Architectures: RetNet and the Three Computation Paradigms",
// section 4.3; the paper summary, Eq. 5), with q', k' the rotated inputs:
//   dq'_n = sum_{m<=n} gamma^(n-m) (dO_n . v_m) k'_m      retention of (q, k, v) = (dO, V, K')
//   dv_m  = sum_{n>=m} gamma^(n-m) (q'_n . k'_m) dO_n     retention of (K', Q', dO) over the reversed sequence
//   dk'_m = sum_{n>=m} gamma^(n-m) (dO_n . v_m) q'_n      retention of (V, dO, Q') over the reversed sequence
// and dq, dk are dq', dk' turned back by the transpose rotation. The forward chunkwise kernels compute the three
// retentions; this kernel prepares their inputs (rotated, reversed) in one launch and finishes their outputs
// (reversed back, rotated back) in another.
#include "kernels.h"

namespace ret {

namespace {

// One thread: one 16-byte segment (8 values, 4 rotation pairs) of kPermTokens consecutive tokens' rows of one
// job (blockIdx.y: the job's fields are scalar loads). Its loads are issued together; the rotation factors of
// the first token are evaluated exactly and carried to the next by angle addition with the one-token step.
// Consecutive threads take consecutive segments of a row, and a job with two outputs writes both from one read.
// Every value is read and written once per launch: the accesses carry the non-temporal hint.
__device__ __forceinline__ void perm_load(const void* p, bool bf16, long long i, float* x) {
    if (bf16) {
        const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>((const uint16_t*)p + i));
        unpack8_bf16(make_uint4(t[0], t[1], t[2], t[3]), x);
    } else {
        const f32x4_t u = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>((const float*)p + i));
        const f32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>((const float*)p + i + 4));
        x[0] = u[0], x[1] = u[1], x[2] = u[2], x[3] = u[3], x[4] = w[0], x[5] = w[1], x[6] = w[2], x[7] = w[3];
    }
}

__device__ __forceinline__ void perm_store(const PermJob& J, void* out, long long i, const float* x) {
    if (J.out_bf16) {
        const uint4 t = pack8_bf16(x);
        __builtin_nontemporal_store(u32x4_t{t.x, t.y, t.z, t.w}, reinterpret_cast<u32x4_t*>((uint16_t*)out + i));
    } else {
        __builtin_nontemporal_store(f32x4_t{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4_t*>((float*)out + i));
        __builtin_nontemporal_store(f32x4_t{x[4], x[5], x[6], x[7]}, reinterpret_cast<f32x4_t*>((float*)out + i + 4));
    }
}

__global__ __launch_bounds__(256) void permute_rotate_kernel(PermArgs a) {
    const PermJob J = a.job[blockIdx.y];
    const unsigned segs = (unsigned)(a.H * J.d / 8);  // segments of one token's row: h * d / 8 + s
    const unsigned gid = blockIdx.x * 256u + threadIdx.x;
    const unsigned nblk = (unsigned)((a.N + kPermTokens - 1) / kPermTokens);
    const unsigned blk = gid / segs, sj = gid - blk * segs;
    if (blk >= (unsigned)a.B * nblk) return;
    const int b = (int)(blk / nblk), t0 = (int)(blk - (unsigned)b * nblk) * kPermTokens;
    const int nt = min(kPermTokens, a.N - t0);
    const long long rowlen = (long long)a.H * J.d;
    const unsigned col = sj * 8u;
    const long long base = (long long)b * a.N * rowlen + col;
    // input: columns col0 .. col0 + d - 1 of each head of width d_in
    const int din = J.d_in ? J.d_in : J.d;
    const unsigned hh = col / (unsigned)J.d, cc = col - hh * (unsigned)J.d;
    const long long rowlen_in = (long long)a.H * din;
    const long long ibase = (long long)b * a.N * rowlen_in + (long long)hh * din + J.col0 + cc;
    float x[kPermTokens][8];
#pragma unroll
    for (int i = 0; i < kPermTokens; ++i)
        if (i < nt) perm_load(J.in, J.in_bf16, ibase + (J.in_rev ? a.N - 1 - (t0 + i) : t0 + i) * rowlen_in, x[i]);
    if (J.in2) {
#pragma unroll
        for (int i = 0; i < kPermTokens; ++i)
            if (i < nt) {
                float y[8];
                perm_load(J.in2, J.in_bf16, ibase + (J.in_rev ? a.N - 1 - (t0 + i) : t0 + i) * rowlen_in, y);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[i][e] += y[e];
            }
    }
    if (J.rot) {
        const int pair0 = (int)(col % (unsigned)J.d) / 2;
        float c[4], s[4], dc[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            rot_cs(a.pos0 + t0, a.theta[pair0 + e], &c[e], &s[e]);
            rot_cs(1, a.theta[pair0 + e], &dc[e], &ds[e]);
            if (J.rot < 0) s[e] = -s[e], ds[e] = -ds[e];  // the transpose rotation
        }
#pragma unroll
        for (int i = 0; i < kPermTokens; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x0 = x[i][2 * e], x1 = x[i][2 * e + 1];
                x[i][2 * e] = x0 * c[e] - x1 * s[e];
                x[i][2 * e + 1] = x0 * s[e] + x1 * c[e];
                const float nc = c[e] * dc[e] - s[e] * ds[e];
                s[e] = s[e] * dc[e] + c[e] * ds[e];
                c[e] = nc;
            }
        }
    }
#pragma unroll
    for (int o = 0; o < 2; ++o) {
        if (!J.out[o]) continue;
#pragma unroll
        for (int i = 0; i < kPermTokens; ++i)
            if (i < nt) perm_store(J, J.out[o], base + (J.out_rev[o] ? a.N - 1 - (t0 + i) : t0 + i) * rowlen, x[i]);
    }
}

__global__ __launch_bounds__(256) void zero_words_kernel(int* p, long long n) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0;
}

}  // namespace

perm_kernel_t permute_rotate_get() { return permute_rotate_kernel; }
zero_kernel_t zero_words_get() { return zero_words_kernel; }

}  // namespace ret
