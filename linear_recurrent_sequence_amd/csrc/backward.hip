// Reordering and rotation of [B, N, H, d] tensors for the gradients of chunkwise retention.
//
// The gradients of L = sum(dO (.) O), O the retention output from a zero state, are themselves retentions
// (they follow from the parallel form, "Hybrid Architectures: RetNet and the Three Computation Paradigms",
// section 4.3; the paper summary, Eq. 5), with q', k' the rotated inputs:
//   dq'_n = sum_{m<=n} gamma^(n-m) (dO_n . v_m) k'_m      retention of (q, k, v) = (dO, V, K')
//   dv_m  = sum_{n>=m} gamma^(n-m) (q'_n . k'_m) dO_n     retention of (K', Q', dO) over the reversed sequence
//   dk'_m = sum_{n>=m} gamma^(n-m) (dO_n . v_m) q'_n      retention of (V, dO, Q') over the reversed sequence
// and dq, dk are dq', dk' turned back by the transpose rotation. The forward chunkwise kernels compute the three
// retentions; this kernel prepares their inputs (rotated, reversed) and finishes their outputs (reversed back,
// rotated back).
#include "kernels.h"

namespace ret {

namespace {

// One thread: 8 consecutive dims (4 rotation pairs) of one output row. Output row (b, n, h) is token
// t = out_rev ? N-1-n : n; it is read from input row in_rev ? N-1-t : t and turned by rot_sign (pos0 + t) theta_i.
__global__ __launch_bounds__(256) void permute_rotate_kernel(PermArgs a) {
    const int segs = a.d / 8;
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long rows = (long long)a.B * a.N * a.H;
    if (gid >= rows * segs) return;
    const int sg = (int)(gid % segs);
    const long long row = gid / segs;  // ((b * N) + n) * H + h
    const int h = (int)(row % a.H);
    const long long bn = row / a.H;
    const int n = (int)(bn % a.N);
    const long long b = bn / a.N;
    const int t = a.out_rev ? a.N - 1 - n : n;
    const int src = a.in_rev ? a.N - 1 - t : t;
    const long long ii = ((b * a.N + src) * a.H + h) * a.d + sg * 8;
    const long long oi = row * a.d + sg * 8;
    float x[8];
    if (a.in_bf16) {
        unpack8_bf16(*reinterpret_cast<const uint4*>((const uint16_t*)a.in + ii), x);
    } else {
        const float4 u = *reinterpret_cast<const float4*>((const float*)a.in + ii);
        const float4 w = *reinterpret_cast<const float4*>((const float*)a.in + ii + 4);
        x[0] = u.x, x[1] = u.y, x[2] = u.z, x[3] = u.w, x[4] = w.x, x[5] = w.y, x[6] = w.z, x[7] = w.w;
    }
    if (a.rot_sign) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float c, s;
            rot_cs(a.pos0 + t, a.theta[sg * 4 + j], &c, &s);
            if (a.rot_sign < 0) s = -s;  // the transpose rotation
            const float x0 = x[2 * j], x1 = x[2 * j + 1];
            x[2 * j] = x0 * c - x1 * s;
            x[2 * j + 1] = x0 * s + x1 * c;
        }
    }
    if (a.out_bf16) {
        *reinterpret_cast<uint4*>((uint16_t*)a.out + oi) = pack8_bf16(x);
    } else {
        *reinterpret_cast<float4*>((float*)a.out + oi) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4*>((float*)a.out + oi + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
}

}  // namespace

perm_kernel_t permute_rotate_get() { return permute_rotate_kernel; }

}  // namespace ret
