// Parallel-form, decode-step and segment-scan kernel instances.
#include "kernels.h"

namespace ret {

// ---------------------------------------------------------------------------------------------------
// segment_scan: per (b, h), W[0] = state_in (or 0); W[g] = gamma^seg_len W[g-1] + W[g] for g = 1..nseg-1,
// where W[g] held the local end state of segment g - 1. Elementwise over d_k x d_v, sequential over g.
// ---------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void segment_scan_kernel(FwdArgs a) {
    const int pair = blockIdx.y;
    const long long per = (long long)a.dk * a.dv;
    const long long e = ((long long)blockIdx.x * kThreads + threadIdx.x) * 4;
    if (e >= per) return;
    const float decay = gpow(a.log2g[pair % a.H], (float)a.seg_len);
    float* W = a.ws + (long long)pair * a.nseg * per;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.state_in) acc = *reinterpret_cast<const float4*>(a.state_in + (long long)pair * per + e);
    *reinterpret_cast<float4*>(W + e) = acc;
    for (int g = 1; g < a.nseg; ++g) {
        float4 u = *reinterpret_cast<const float4*>(W + (long long)g * per + e);
        acc.x = decay * acc.x + u.x;
        acc.y = decay * acc.y + u.y;
        acc.z = decay * acc.z + u.z;
        acc.w = decay * acc.w + u.w;
        *reinterpret_cast<float4*>(W + (long long)g * per + e) = acc;
    }
}

bool parallel_kernel_get(bool bf16_in, int dk, int dv, ParKernel* out) {
    if (!bf16_in) {
        if (dv % 16) return false;
        if (dk == 16) { *out = {parallel_kernel<F32, 16, 32, 16>, 32, 16}; return true; }
        if (dk == 32) { *out = {parallel_kernel<F32, 32, 32, 16>, 32, 16}; return true; }
        if (dk == 64) { *out = {parallel_kernel<F32, 64, 32, 16>, 32, 16}; return true; }
        return false;
    }
    if (dv % 64) return false;
    if (dk == 32) { *out = {parallel_kernel<BF16, 32, 64, 64>, 64, 64}; return true; }
    if (dk == 64) { *out = {parallel_kernel<BF16, 64, 64, 64>, 64, 64}; return true; }
    if (dk == 128) { *out = {parallel_kernel<BF16, 128, 64, 64>, 64, 64}; return true; }
    if (dk == 256) { *out = {parallel_kernel<BF16, 256, 64, 64>, 64, 64}; return true; }
    return false;
}

step_kernel_t step_kernel_get(int dk) {
    switch (dk) {
        case 16: return recurrent_step_kernel<16>;
        case 32: return recurrent_step_kernel<32>;
        case 64: return recurrent_step_kernel<64>;
        case 128: return recurrent_step_kernel<128>;
        case 256: return recurrent_step_kernel<256>;
        default: return nullptr;
    }
}

fwd_kernel_t segment_scan_get() { return segment_scan_kernel; }

}  // namespace ret
