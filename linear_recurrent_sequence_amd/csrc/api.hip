// C ABI of libretention.so: argument validation, kernel selection, segment planning, launches and the
// optional kernel-timing records. Sources for each operation are cited in retention.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "retention.h"

// =====================================================================================================
// Host side: validation, kernel selection, launches, timing records.
// =====================================================================================================
namespace {

using namespace ret;

thread_local std::string g_last_error;

ret_status_t fail(ret_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ret_status_t fail(ret_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

// ---- timing records ----
struct TimingRec {
    const char* name;
    hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<TimingRec> g_timing;

struct LaunchTimer {
    hipEvent_t start = nullptr, stop = nullptr;
    hipStream_t stream;
    const char* name;
    bool on;
    LaunchTimer(const char* n, hipStream_t s) : stream(s), name(n) {
        {
            std::lock_guard<std::mutex> lk(g_timing_mu);
            on = g_timing_on;
        }
        if (on && hipEventCreate(&start) == hipSuccess && hipEventCreate(&stop) == hipSuccess)
            (void)hipEventRecord(start, stream);
        else
            on = false;
    }
    void done() {
        if (!on) return;
        (void)hipEventRecord(stop, stream);
        std::lock_guard<std::mutex> lk(g_timing_mu);
        g_timing.push_back({name, start, stop});
    }
};

ret_status_t launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(RET_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return RET_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

ret_status_t check_common(const void* q, const void* k, const void* v, void* o, int B, int N, int H, int dk, int dv,
                          ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma, const double* theta) {
    if (!q || !k || !v || !o) return fail(RET_ERR_INVALID_ARG, "null q/k/v/o pointer");
    if (B <= 0 || N <= 0 || H <= 0 || dk <= 0 || dv <= 0)
        return fail(RET_ERR_INVALID_ARG, "sizes must be positive (B=%d N=%d H=%d dk=%d dv=%d)", B, N, H, dk, dv);
    if (!gamma) return fail(RET_ERR_INVALID_ARG, "null gamma");
    if (in_dt != RET_F32 && in_dt != RET_BF16) return fail(RET_ERR_INVALID_ARG, "bad in_dt %d", (int)in_dt);
    if (out_dt != RET_F32 && out_dt != RET_BF16) return fail(RET_ERR_INVALID_ARG, "bad out_dt %d", (int)out_dt);
    if (in_dt == RET_F32 && out_dt != RET_F32)
        return fail(RET_ERR_INVALID_ARG, "F32 input requires F32 output");
    if (H > kMaxHeads) return fail(RET_ERR_UNSUPPORTED, "H=%d exceeds %d heads", H, kMaxHeads);
    if ((long long)B * H > 65535) return fail(RET_ERR_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)B * H);
    for (int h = 0; h < H; ++h)
        if (!(gamma[h] > 0.f && gamma[h] <= 1.f))
            return fail(RET_ERR_INVALID_ARG, "gamma[%d]=%g outside (0, 1]", h, (double)gamma[h]);
    if (theta) {
        if (dk % 2) return fail(RET_ERR_INVALID_ARG, "rotation needs an even d_k (got %d)", dk);
        if (dk / 2 > kMaxPairs) return fail(RET_ERR_UNSUPPORTED, "rotation supports d_k <= %d", 2 * kMaxPairs);
        for (int i = 0; i < dk / 2; ++i)
            if (!isfinite(theta[i])) return fail(RET_ERR_INVALID_ARG, "theta[%d] is not finite", i);
    }
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(RET_ERR_INVALID_ARG, "q/k/v/o must be 16-byte aligned");
    if (o == q || o == k || o == v) return fail(RET_ERR_INVALID_ARG, "o must not alias q, k or v");
    return RET_OK;
}

void fill_fwd(FwdArgs& A, const void* q, const void* k, const void* v, void* o, int B, int N, int H, int dk, int dv,
              ret_dtype_t out_dt, const float* gamma, const double* theta, int64_t pos0) {
    memset(&A, 0, sizeof(A));
    A.q = q;
    A.k = k;
    A.v = v;
    A.o = o;
    A.B = B;
    A.N = N;
    A.H = H;
    A.dk = dk;
    A.dv = dv;
    A.out_bf16 = out_dt == RET_BF16;
    A.rotate = theta != nullptr;
    A.pos0 = pos0;
    for (int h = 0; h < H; ++h) A.log2g[h] = (float)log2((double)gamma[h]);
    if (theta)
        for (int i = 0; i < dk / 2; ++i) A.theta[i] = theta[i];
}

// ---- kernel selection ----
bool pick_chunk(ret_dtype_t in_dt, int dk, int dv, int C, ChunkKernels* out) {
    if (in_dt == RET_F32) return chunk_kernels_f32(dk, dv, C, out);
    if (dk == 32 || dk == 64) return chunk_kernels_bf16_small(dk, dv, C, out);
    if (dk == 128) return chunk_kernels_bf16_128(dk, dv, C, out);
    if (dk == 256) return chunk_kernels_bf16_256(dk, dv, C, out);
    return false;
}

bool pick_parallel(ret_dtype_t in_dt, int dk, int dv, ParKernel* out) {
    return parallel_kernel_get(in_dt == RET_BF16, dk, dv, out);
}

// ---- segment heuristic ----
int env_int(const char* name, int dflt) {
    const char* s = getenv(name);
    if (!s || !*s) return dflt;
    return atoi(s);
}

// Number of segments per sequence and tokens per segment. Enough workgroups to fill the chip, but segments of
// at least ~256 tokens so the per-segment state traffic stays small against the segment's own data.
void plan_segments(int B, int N, int H, int dv, int C, int dvt, int target_wgs, int* nseg, int* seg_len) {
    const long long units = (long long)B * H * ((dv + dvt - 1) / dvt);
    const int nchunks = (N + C - 1) / C;
    const int target = env_int("RET_TARGET_WGS", target_wgs > 0 ? target_wgs : 1024);
    int g = (int)((target + units - 1) / units);
    const int forced = env_int("RET_SEGMENTS", 0);
    if (forced > 0) g = forced;
    if (g < 1) g = 1;
    if (g > nchunks) g = nchunks;
    int spc = (nchunks + g - 1) / g;  // chunks per segment
    const int min_spc = forced > 0 ? 1 : (256 + C - 1) / C;
    if (spc < min_spc) spc = min_spc;
    if (spc > nchunks) spc = nchunks;
    *seg_len = spc * C;
    *nseg = (nchunks + spc - 1) / spc;
}

// Workspace bytes for nseg segments: the chain layout for the single-pass kernels, else one end state per
// (sequence, segment) for the split kernels.
size_t segment_ws_bytes(const ChunkKernels& ck, int B, int H, int dk, int dv, int nseg) {
    if (nseg <= 1) return 0;
    if (ck.fused) return chain_layout(B * H * (dv / ck.dvt), nseg, dk * ck.dvt).bytes;
    return sizeof(ChainHeader) + (size_t)B * H * nseg * dk * dv * sizeof(float);
}

// The plan of one chunkwise call: segments, and whether q and k are rotated once up front into the workspace
// (bf16 single-pass kernels with at least 4 d_v tiles, i.e. staging would rotate the same rows 4+ times).
// Workspace layout: [segment chain or split-kernel states][q'][k'], each part 256-byte aligned. A smaller
// workspace first drops the rotated copies, then halves the segment count until the states fit.
struct ChunkPlan {
    int nseg, seg_len;
    size_t chain_bytes, rot_bytes;
};
ChunkPlan plan_chunk(const ChunkKernels& ck, int B, int N, int H, int dk, int dv, int chunk, bool rotate,
                     size_t avail) {
    ChunkPlan p;
    plan_segments(B, N, H, dv, chunk, ck.dvt, ck.target_wgs, &p.nseg, &p.seg_len);
    p.chain_bytes = (segment_ws_bytes(ck, B, H, dk, dv, p.nseg) + 255) / 256 * 256;
    p.rot_bytes = 0;
    // RET_PREROTATE=0 / 1 turns the up-front rotation off / on wherever a kernel supports it.
    const int pre = env_int("RET_PREROTATE", -1);
    if (ck.fused_pre && rotate && (pre < 0 ? dv / ck.dvt >= 4 : pre != 0))
        p.rot_bytes = 2 * (((size_t)B * N * H * dk * 2 + 255) / 256 * 256);
    if (p.chain_bytes + p.rot_bytes > avail) p.rot_bytes = 0;
    while (p.nseg > 1 && segment_ws_bytes(ck, B, H, dk, dv, p.nseg) > avail) {
        const int nchunks = (N + chunk - 1) / chunk;
        int spc = p.seg_len / chunk * 2;
        if (spc > nchunks) spc = nchunks;
        p.seg_len = spc * chunk;
        p.nseg = (nchunks + spc - 1) / spc;
        p.chain_bytes = (segment_ws_bytes(ck, B, H, dk, dv, p.nseg) + 255) / 256 * 256;
    }
    if (p.nseg == 1) {
        p.seg_len = N;
        p.chain_bytes = 0;
    }
    return p;
}

// Whether a plan runs the on-chip segment kernel: chained segments short enough to stay on chip
// (RET_SEG_ONCHIP=0 turns it off).
bool plan_onchip(const ChunkKernels& ck, const ChunkPlan& p) {
    return ck.fused && p.nseg > 1 && ck.seg && p.seg_len <= ck.seg_tokens && env_int("RET_SEG_ONCHIP", 1) != 0;
}

}  // namespace

// =====================================================================================================
// Exported C ABI
// =====================================================================================================
extern "C" {

int ret_abi_version(void) { return RET_ABI_VERSION; }

const char* ret_status_string(int status) {
    switch (status) {
        case RET_OK: return "ok";
        case RET_ERR_INVALID_ARG: return "invalid argument";
        case RET_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case RET_ERR_WORKSPACE: return "workspace too small or missing";
        case RET_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* ret_last_error(void) { return g_last_error.c_str(); }

ret_status_t ret_parallel_fwd(const void* q, const void* k, const void* v, void* o, int B, int N, int H, int dk,
                              int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                              const double* theta, int64_t pos0, void* stream) {
    ret_status_t st = check_common(q, k, v, o, B, N, H, dk, dv, in_dt, out_dt, gamma, theta);
    if (st != RET_OK) return st;
    ParKernel pk;
    if (!pick_parallel(in_dt, dk, dv, &pk))
        return fail(RET_ERR_UNSUPPORTED, "parallel form: unsupported d_k=%d d_v=%d for %s input", dk, dv,
                    in_dt == RET_F32 ? "F32" : "BF16");
    FwdArgs A;
    fill_fwd(A, q, k, v, o, B, N, H, dk, dv, out_dt, gamma, theta, pos0);
    hipStream_t s = (hipStream_t)stream;
    dim3 grid((N + pk.bq - 1) / pk.bq, dv / pk.dvt, B * H);
    LaunchTimer tm("ret_parallel", s);
    hipLaunchKernelGGL(pk.fn, grid, dim3(kThreads), 0, s, A);
    tm.done();
    return launch_status("ret_parallel");
}

size_t ret_chunkwise_workspace_bytes(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt) {
    ChunkKernels ck;
    if (B <= 0 || N <= 0 || H <= 0 || dk <= 0 || dv <= 0 || chunk <= 0) return 0;
    if (!pick_chunk(in_dt, dk, dv, chunk, &ck)) return 0;
    const ChunkPlan p = plan_chunk(ck, B, N, H, dk, dv, chunk, true, SIZE_MAX);
    return p.chain_bytes + p.rot_bytes;
}

}  // extern "C"

namespace {

// The epilogue a chunkwise call may fuse into its output stores.
struct EpiRequest {
    const void* gate;
    ret_dtype_t gate_dt;
    const float *weight, *bias;
    float eps;
};

// ret_chunkwise_fwd's work. With `epi`, the kernel applies the epilogue to the outputs before storing them where
// it holds whole head rows (the on-chip kernel with bf16 output and d_v = 64), and *fused says whether it did.
ret_status_t chunkwise_run(const void* q, const void* k, const void* v, void* o, int B, int N, int H, int dk,
                           int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma, const double* theta,
                           int64_t pos0, int chunk, const float* state_in, float* state_out, void* workspace,
                           size_t workspace_bytes, void* stream, const EpiRequest* epi, bool* fused,
                           bool rev = false, const double* out_theta = nullptr) {
    if (fused) *fused = false;
    ret_status_t st = check_common(q, k, v, o, B, N, H, dk, dv, in_dt, out_dt, gamma, theta);
    if (st != RET_OK) return st;
    if (chunk <= 0) return fail(RET_ERR_INVALID_ARG, "chunk must be positive (got %d)", chunk);
    if ((state_in && !aligned16(state_in)) || (state_out && !aligned16(state_out)))
        return fail(RET_ERR_INVALID_ARG, "state buffers must be 16-byte aligned");
    if (workspace_bytes > 0 && !workspace) return fail(RET_ERR_WORKSPACE, "workspace_bytes > 0 with a null workspace");
    if (workspace && !aligned16(workspace)) return fail(RET_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    ChunkKernels ck;
    if (!pick_chunk(in_dt, dk, dv, chunk, &ck))
        return fail(RET_ERR_UNSUPPORTED, "chunkwise form: unsupported d_k=%d d_v=%d chunk=%d for %s input", dk, dv,
                    chunk, in_dt == RET_F32 ? "F32" : "BF16");
    if (rev && !ck.fused) return fail(RET_ERR_UNSUPPORTED, "reversed chunkwise run: not available for this shape");
    // The kernels address one chunk of one head with 32-bit byte offsets.
    if ((long long)chunk * H * (dk > dv ? dk : dv) * 4 >= (1LL << 31))
        return fail(RET_ERR_UNSUPPORTED, "chunkwise form: chunk*H*max(d_k,d_v) too large (%d*%d*%d)", chunk, H,
                    dk > dv ? dk : dv);
    const ChunkPlan plan = plan_chunk(ck, B, N, H, dk, dv, chunk, theta != nullptr, workspace_bytes);
    const int nseg = plan.nseg, seg_len = plan.seg_len;

    FwdArgs A;
    fill_fwd(A, q, k, v, o, B, N, H, dk, dv, out_dt, gamma, theta, pos0);
    A.state_in = state_in;
    A.state_out = state_out;
    // The split kernels keep their segment states after the (unused, zero) chain header.
    A.ws = ck.fused || !workspace ? (float*)workspace : (float*)((char*)workspace + sizeof(ChainHeader));
    A.nseg = nseg;
    A.seg_len = seg_len;
    hipStream_t s = (hipStream_t)stream;
    const int ntiles = dv / ck.dvt;
    if (ck.fused) {
        // Segments short enough to stay on chip take the on-chip variant.
        const bool onchip = plan_onchip(ck, plan);
        // Staging copies rows instead of rotating them when there is no rotation, or when q and k are rotated
        // once up front (several d_v tiles stage the same rows).
        fwd_kernel_t fn = onchip ? ck.seg : ck.fused;
        const fwd_kernel_t fn_pre = onchip ? (rev ? ck.seg_rev : ck.seg_pre) : ck.fused_pre;
        // the reversed run and the rotation of the outputs exist for the on-chip kernel without input rotation,
        // state or epilogue only
        if ((rev || out_theta) && (!onchip || (rev && !ck.seg_rev) || theta || state_in || state_out || epi))
            return fail(RET_ERR_UNSUPPORTED, "reversed or output-rotated chunkwise run: not available for this shape");
        if (out_theta) {
            A.orot = 1;
            for (int i = 0; i < dv / 2; ++i) A.theta[i] = out_theta[i];
        }
        const char* name = onchip ? "ret_chunk_seg" : "ret_chunk_fused";
        if (!theta) {
            fn = fn_pre;
            A.qr = const_cast<void*>(q);
            A.kr = const_cast<void*>(k);
        } else if (plan.rot_bytes > 0) {
            fn = fn_pre;
            A.qr = (char*)workspace + plan.chain_bytes;
            A.kr = (char*)A.qr + plan.rot_bytes / 2;
            LaunchTimer tr("ret_rotate_qk", s);
            hipLaunchKernelGGL(rotate_qk_get(), dim3(rotate_qk_blocks(B, N, H, dk)), dim3(256), 0, s, A);
            tr.done();
            if ((st = launch_status("ret_rotate_qk")) != RET_OK) return st;
        }
        const unsigned grid = (unsigned)((long long)nseg * B * H * ntiles);
        const int threads = onchip || !ck.threads ? kThreads : ck.threads;
        if (epi && onchip && out_dt == RET_BF16 && dv == 64) {
            A.epi = 1;
            A.gate = epi->gate;
            A.gate_bf16 = epi->gate_dt == RET_BF16;
            A.gn_weight = epi->weight;
            A.gn_bias = epi->bias;
            A.eps = epi->eps;
            if (fused) *fused = true;
        }
        LaunchTimer tm(name, s);
        hipLaunchKernelGGL(fn, dim3(grid), dim3(threads), 0, s, A);
        tm.done();
        return launch_status(name);
    }
    if (nseg > 1) {
        {
            LaunchTimer tm("ret_chunk_local", s);
            hipLaunchKernelGGL(ck.local, dim3(nseg - 1, ntiles, B * H), dim3(kThreads), 0, s, A);
            tm.done();
            if ((st = launch_status("ret_chunk_local")) != RET_OK) return st;
        }
        {
            const long long per4 = (long long)dk * dv / 4;
            LaunchTimer tm("ret_segment_scan", s);
            hipLaunchKernelGGL(segment_scan_get(), dim3((unsigned)((per4 + kThreads - 1) / kThreads), B * H),
                               dim3(kThreads), 0, s, A);
            tm.done();
            if ((st = launch_status("ret_segment_scan")) != RET_OK) return st;
        }
    }
    LaunchTimer tm("ret_chunk_full", s);
    hipLaunchKernelGGL(ck.full, dim3(nseg, ntiles, B * H), dim3(kThreads), 0, s, A);
    tm.done();
    return launch_status("ret_chunk_full");
}

// Workspace of the gradients. At offset 0 the segment chain the three retentions share (one call after
// another; at least 256 bytes, so ret_chunkwise_check reads its header). Then, when both reversed retentions run
// on the on-chip kernel's reversed traversal (direct, bf16 only): Q' and K' (bf16, only with rotation). Otherwise the reordered inputs K', K' reversed, Q' reversed, V reversed, dO reversed (in
// the input dtype) and the three fp32 outputs.
struct BwdLayout {
    bool direct;
    int nb, wb;  // d_v blocks of width wb for the retentions that contract over d_v (nb = 2 when d_v is wider
                 // than their kernels' d_k; dq' and dk' are then sums of two retentions)
    size_t qp, kp, kr, qr, vr, dor, g1, g2, g3, chain, chain_bytes, total;
    size_t vbn[2], dobn[2], vbr[2], dobr[2], g1b[2], g3b[2];  // per block (nb = 2)
};
bool bwd_layout(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt, bool rotate, BwdLayout* L) {
    ChunkKernels ca, cb;
    memset(L, 0, sizeof(*L));
    L->nb = 1;
    L->wb = dv;
    if (!pick_chunk(in_dt, dv, dk, chunk, &ca)) {
        // d_v too wide to be the contraction width of a retention: two halves, each a retention of its own
        if (dv % 2 || (dv / 2) % 16 || !pick_chunk(in_dt, dv / 2, dk, chunk, &ca)) return false;
        L->nb = 2;
        L->wb = dv / 2;
    }
    if (!pick_chunk(in_dt, dk, dv, chunk, &cb)) return false;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t nk = (size_t)B * N * H * dk, nv = (size_t)B * N * H * dv, es = in_dt == RET_BF16 ? 2 : 4;
    const size_t nw = (size_t)B * N * H * L->wb;
    const ChunkPlan pa = plan_chunk(ca, B, N, H, L->wb, dk, chunk, false, SIZE_MAX);
    const ChunkPlan pb = plan_chunk(cb, B, N, H, dk, dv, chunk, false, SIZE_MAX);
    L->direct = in_dt == RET_BF16 && L->nb == 1 && plan_onchip(ca, pa) && ca.seg_rev && plan_onchip(cb, pb) &&
                cb.seg_rev && env_int("RET_BWD_DIRECT", 1) != 0;
    L->chain = 0;
    L->chain_bytes = pa.chain_bytes > pb.chain_bytes ? pa.chain_bytes : pb.chain_bytes;
    size_t off = up(L->chain_bytes > 256 ? L->chain_bytes : 256);
    if (L->direct) {
        if (rotate) {
            L->qp = off;
            L->kp = L->qp + up(nk * 2);
            off = L->kp + up(nk * 2);
        }
        L->total = off;
        return true;
    }
    if (L->nb == 2) {
        L->kp = off;
        L->kr = L->kp + up(nk * es);
        L->qr = L->kr + up(nk * es);
        L->dor = L->qr + up(nk * es);
        off = L->dor + up(nv * es);
        for (int i = 0; i < 2; ++i) {
            L->vbn[i] = off;
            L->dobn[i] = L->vbn[i] + up(nw * es);
            L->vbr[i] = L->dobn[i] + up(nw * es);
            L->dobr[i] = L->vbr[i] + up(nw * es);
            off = L->dobr[i] + up(nw * es);
        }
        for (int i = 0; i < 2; ++i) {
            L->g1b[i] = off;
            L->g3b[i] = L->g1b[i] + up(nk * 4);
            off = L->g3b[i] + up(nk * 4);
        }
        L->g2 = off;
        L->total = L->g2 + up(nv * 4);
        return true;
    }
    L->kp = off;
    L->kr = L->kp + up(nk * es);
    L->qr = L->kr + up(nk * es);
    L->vr = L->qr + up(nk * es);
    L->dor = L->vr + up(nv * es);
    L->g1 = L->dor + up(nv * es);
    L->g2 = L->g1 + up(nk * 4);
    L->g3 = L->g2 + up(nv * 4);
    L->total = L->g3 + up(nk * 4);
    return true;
}

// The gradients' retentions share one segment chain, but calls of different shapes lay it out differently:
// one call's published slots can lie where the next call expects zero counters and flags. Before a call whose
// layout differs from the previous call's, its counters and flags (not the header, which keeps a sticky error)
// are zeroed by a small kernel (graph-safe, unlike a memset node).
ret_status_t chain_meta_zero(ret_dtype_t in_dt, int B, int N, int H, int dk, int dv, int chunk, void* chain,
                             size_t chain_bytes, hipStream_t s) {
    ChunkKernels ck;
    if (!pick_chunk(in_dt, dk, dv, chunk, &ck) || !ck.fused) return RET_OK;  // the split kernels keep no flags
    const ChunkPlan p = plan_chunk(ck, B, N, H, dk, dv, chunk, false, chain_bytes);
    if (p.nseg <= 1) return RET_OK;
    const ChainLayout lay = chain_layout(B * H * (dv / ck.dvt), p.nseg, dk * ck.dvt);
    const long long n = (long long)(lay.agg_off - lay.ctr_off) / 4;
    hipLaunchKernelGGL(zero_words_get(), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (int*)((char*)chain + lay.ctr_off), n);
    return launch_status("chain_meta_zero");
}

// One launch of permute_rotate_kernel over the given jobs (at most kMaxPermJobs), one grid row per job.
ret_status_t permute(const PermJob* jobs, int njobs, int B, int N, int H, const double* theta, int64_t pos0,
                     hipStream_t s) {
    PermArgs P;
    memset(&P, 0, sizeof(P));
    P.B = B;
    P.N = N;
    P.H = H;
    P.pos0 = pos0;
    unsigned long long segs = 0;
    for (int j = 0; j < njobs; ++j) {
        P.job[j] = jobs[j];
        if (!theta) P.job[j].rot = 0;
        const unsigned long long sj = (unsigned long long)H * jobs[j].d / 8;
        if (sj > segs) segs = sj;
    }
    if (theta)
        for (int i = 0; i < kMaxPairs; ++i) P.theta[i] = i < jobs[0].d / 2 ? theta[i] : 0.0;
    const unsigned long long threads = (unsigned long long)B * ((N + kPermTokens - 1) / kPermTokens) * segs;
    if ((long long)B * N >= (1LL << 31) || threads > 0xFFFFFF00ull)
        return fail(RET_ERR_UNSUPPORTED, "gradients: B*N*H*max(d_k,d_v) too large for one reordering launch");
    LaunchTimer tm("ret_permute_rotate", s);
    hipLaunchKernelGGL(permute_rotate_get(), dim3((unsigned)((threads + 255) / 256), njobs), dim3(256), 0, s, P);
    tm.done();
    return launch_status("ret_permute_rotate");
}

}  // namespace

extern "C" {

ret_status_t ret_chunkwise_fwd(const void* q, const void* k, const void* v, void* o, int B, int N, int H, int dk,
                               int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                               const double* theta, int64_t pos0, int chunk, const float* state_in,
                               float* state_out, void* workspace, size_t workspace_bytes, void* stream) {
    return chunkwise_run(q, k, v, o, B, N, H, dk, dv, in_dt, out_dt, gamma, theta, pos0, chunk, state_in, state_out,
                         workspace, workspace_bytes, stream, nullptr, nullptr);
}

ret_status_t ret_chunkwise_msr_fwd(const void* q, const void* k, const void* v, const void* gate, void* y, int B,
                                   int N, int H, int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt,
                                   ret_dtype_t gate_dt, const float* gamma, const double* theta, int64_t pos0,
                                   int chunk, const float* state_in, float* state_out, const float* gn_weight,
                                   const float* gn_bias, float eps, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    // The epilogue's own checks first, so that nothing is launched for a call that would fail half way.
    if (gate_dt != RET_F32 && gate_dt != RET_BF16) return fail(RET_ERR_INVALID_ARG, "bad gate dtype %d", (int)gate_dt);
    if (!(eps >= 0.f) || !isfinite(eps)) return fail(RET_ERR_INVALID_ARG, "eps=%g must be finite and >= 0", eps);
    if ((gate && !aligned16(gate)) || (gn_weight && !aligned16(gn_weight)) || (gn_bias && !aligned16(gn_bias)))
        return fail(RET_ERR_INVALID_ARG, "gate/gn_weight/gn_bias must be 16-byte aligned");
    int gpw = 0;
    if (!epilogue_kernel_get(dv, &gpw))
        return fail(RET_ERR_UNSUPPORTED, "epilogue: d_v=%d not in {16,32,64,128,256,512}", dv);
    if (gate && (gate == q || gate == k || gate == v || gate == y))
        return fail(RET_ERR_INVALID_ARG, "gate must not alias q, k, v or y");
    if ((long long)B * N * H > 0x7fffffffLL)
        return fail(RET_ERR_UNSUPPORTED, "epilogue: B*N*H=%lld exceeds 2^31 groups", (long long)B * N * H);
    const EpiRequest epi{gate, gate_dt, gn_weight, gn_bias, eps};
    bool fused = false;
    ret_status_t st = chunkwise_run(q, k, v, y, B, N, H, dk, dv, in_dt, out_dt, gamma, theta, pos0, chunk, state_in,
                                    state_out, workspace, workspace_bytes, stream, &epi, &fused);
    if (st != RET_OK || fused) return st;
    // not fused: the retention outputs are in y; the epilogue runs over them in place
    return ret_msr_epilogue(y, gate, gn_weight, gn_bias, y, (int64_t)B * N, H, dv, out_dt, gate_dt, out_dt, eps,
                            stream);
}

}  // extern "C"

namespace {

// One decode step; positions either one for the call (`pos`) or one per sequence (`pos_dev`, device [B]).
ret_status_t step_run(const void* q, const void* k, const void* v, void* o, float* state, int B, int H, int dk,
                      int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma, const double* theta,
                      int64_t pos, const int64_t* pos_dev, void* stream) {
    ret_status_t st = check_common(q, k, v, o, B, 1, H, dk, dv, in_dt, out_dt, gamma, theta);
    if (st != RET_OK) return st;
    if (!state) return fail(RET_ERR_INVALID_ARG, "null state");
    if (!aligned16(state)) return fail(RET_ERR_INVALID_ARG, "state must be 16-byte aligned");
    if (dv % 4 || dv > 512) return fail(RET_ERR_UNSUPPORTED, "decode step: d_v must be a multiple of 4, <= 512");
    StepArgs A;
    memset(&A, 0, sizeof(A));
    A.q = q;
    A.k = k;
    A.v = v;
    A.o = o;
    A.state = state;
    A.B = B;
    A.H = H;
    A.dk = dk;
    A.dv = dv;
    A.in_bf16 = in_dt == RET_BF16;
    A.out_bf16 = out_dt == RET_BF16;
    A.rotate = theta != nullptr;
    for (int h = 0; h < H; ++h) A.gamma[h] = gamma[h];
    // Rotation factors of this step's position, in fp64 (one position per call); with per-sequence positions
    // the kernel makes them from theta.
    A.pos = theta ? (const long long*)pos_dev : nullptr;
    if (theta && pos_dev)
        for (int i = 0; i < dk / 2; ++i) A.theta[i] = theta[i];
    else if (theta)
        for (int i = 0; i < dk / 2; ++i) {
            const double ang = (double)pos * theta[i];
            A.rc[i] = (float)cos(ang);
            A.rs[i] = (float)sin(ang);
        }
    int cw = 0, wr = 0, ppw = 1;
    step_kernel_t fn = step_kernel_get(in_dt == RET_BF16, dk, dv, B * H, env_int("RET_STEP_CW", 0),
                                       env_int("RET_STEP_WR", 0), env_int("RET_STEP_PAIRS", 0), A.pos != nullptr,
                                       &cw, &wr, &ppw);
    if (!fn) return fail(RET_ERR_UNSUPPORTED, "decode step: d_k=%d not in {16,32,64,128,256}", dk);
    hipStream_t s = (hipStream_t)stream;
    LaunchTimer tm("ret_recurrent_step", s);
    hipLaunchKernelGGL(fn, dim3((dv + cw - 1) / cw, (B * H + ppw - 1) / ppw), dim3(64 * (dk / wr) * ppw), 0, s, A);
    tm.done();
    return launch_status("ret_recurrent_step");
}

}  // namespace

extern "C" {

ret_status_t ret_recurrent_step(const void* q, const void* k, const void* v, void* o, float* state, int B, int H,
                                int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                                const double* theta, int64_t pos, void* stream) {
    return step_run(q, k, v, o, state, B, H, dk, dv, in_dt, out_dt, gamma, theta, pos, nullptr, stream);
}

ret_status_t ret_recurrent_step_positions(const void* q, const void* k, const void* v, void* o, float* state, int B,
                                          int H, int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt,
                                          const float* gamma, const double* theta, const int64_t* pos,
                                          void* stream) {
    if (!pos) return fail(RET_ERR_INVALID_ARG, "null pos");
    if ((uintptr_t)pos % 8) return fail(RET_ERR_INVALID_ARG, "pos must be 8-byte aligned");
    return step_run(q, k, v, o, state, B, H, dk, dv, in_dt, out_dt, gamma, theta, 0, pos, stream);
}

ret_status_t ret_msr_epilogue(const void* o, const void* gate, const float* gn_weight, const float* gn_bias,
                              void* y, int64_t rows, int H, int dv, ret_dtype_t o_dt, ret_dtype_t gate_dt,
                              ret_dtype_t y_dt, float eps, void* stream) {
    if (!o || !y) return fail(RET_ERR_INVALID_ARG, "null o/y pointer");
    if (rows < 0 || H <= 0 || dv <= 0)
        return fail(RET_ERR_INVALID_ARG, "sizes must be positive (rows=%lld H=%d dv=%d)", (long long)rows, H, dv);
    for (ret_dtype_t t : {o_dt, gate_dt, y_dt})
        if (t != RET_F32 && t != RET_BF16) return fail(RET_ERR_INVALID_ARG, "bad dtype %d", (int)t);
    if (!(eps >= 0.f) || !isfinite(eps)) return fail(RET_ERR_INVALID_ARG, "eps=%g must be finite and >= 0", eps);
    if (!aligned16(o) || !aligned16(y) || (gate && !aligned16(gate)) || (gn_weight && !aligned16(gn_weight)) ||
        (gn_bias && !aligned16(gn_bias)))
        return fail(RET_ERR_INVALID_ARG, "o/gate/y/gn_weight/gn_bias must be 16-byte aligned");
    int gpw = 0;
    const epi_kernel_t fn = epilogue_kernel_get(dv, &gpw);
    if (!fn) return fail(RET_ERR_UNSUPPORTED, "epilogue: d_v=%d not in {16,32,64,128,256,512}", dv);
    const long long groups = (long long)rows * H;
    if (groups == 0) return RET_OK;
    if (groups > 0x7fffffffLL)
        return fail(RET_ERR_UNSUPPORTED, "epilogue: %lld rows x %d heads exceed 2^31 groups", (long long)rows, H);
    const long long wgs = (groups + gpw - 1) / gpw;
    EpiArgs A;
    A.o = o;
    A.gate = gate;
    A.weight = gn_weight;
    A.bias = gn_bias;
    A.y = y;
    A.groups = groups;
    A.H = H;
    A.dv = dv;
    A.o_bf16 = o_dt == RET_BF16;
    A.gate_bf16 = gate_dt == RET_BF16;
    A.y_bf16 = y_dt == RET_BF16;
    A.eps = eps;
    hipStream_t s = (hipStream_t)stream;
    LaunchTimer tm("ret_msr_epilogue", s);
    hipLaunchKernelGGL(fn, dim3((unsigned)wgs), dim3(256), 0, s, A);
    tm.done();
    return launch_status("ret_msr_epilogue");
}

size_t ret_chunkwise_bwd_workspace_bytes(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt) {
    BwdLayout L;
    if (B <= 0 || N <= 0 || H <= 0 || dk <= 0 || dv <= 0 || chunk <= 0) return 0;
    if (in_dt != RET_F32 && in_dt != RET_BF16) return 0;
    if (!bwd_layout(B, N, H, dk, dv, chunk, in_dt, true, &L)) return 0;
    return L.total;
}

ret_status_t ret_chunkwise_bwd(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk_out,
                               void* dv_out, int B, int N, int H, int dk, int dv, ret_dtype_t in_dt,
                               ret_dtype_t out_dt, const float* gamma, const double* theta, int64_t pos0, int chunk,
                               void* workspace, size_t workspace_bytes, void* stream) {
    ret_status_t st = check_common(q, k, v, dq, B, N, H, dk, dv, in_dt, out_dt, gamma, theta);
    if (st != RET_OK) return st;
    if (!dout || !dk_out || !dv_out) return fail(RET_ERR_INVALID_ARG, "null dout/dk/dv pointer");
    if (!aligned16(dout) || !aligned16(dk_out) || !aligned16(dv_out))
        return fail(RET_ERR_INVALID_ARG, "dout/dq/dk/dv must be 16-byte aligned");
    for (const void* g : {(const void*)dq, (const void*)dk_out, (const void*)dv_out})
        if (g == q || g == k || g == v || g == dout) return fail(RET_ERR_INVALID_ARG, "gradients must not alias inputs");
    if (dq == dk_out || dq == dv_out || dk_out == dv_out) return fail(RET_ERR_INVALID_ARG, "dq, dk, dv must differ");
    if (chunk <= 0) return fail(RET_ERR_INVALID_ARG, "chunk must be positive (got %d)", chunk);
    BwdLayout L;
    if (!bwd_layout(B, N, H, dk, dv, chunk, in_dt, theta != nullptr, &L))
        return fail(RET_ERR_UNSUPPORTED,
                    "gradients: d_k=%d d_v=%d chunk=%d for %s input (both (d_k, d_v) and (d_v, d_k) need kernels)", dk,
                    dv, chunk, in_dt == RET_F32 ? "F32" : "BF16");
    if (!workspace || workspace_bytes < L.total)
        return fail(RET_ERR_WORKSPACE, "gradients need a workspace of %zu bytes (got %zu)", L.total, workspace_bytes);
    if (!aligned16(workspace)) return fail(RET_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    const int ob = out_dt == RET_BF16;
    if (L.direct) {
        // Q', K' (rotated once; q and k themselves without rotation), then dq' = retention(dO, V, K') and, over
        // the reversed sequence on the reversed traversal, dv = retention(K', Q', dO) and dk' = retention(V, dO,
        // Q'), written in token order; dq' and dk' leave their kernels turned back by the transpose rotation.
        const void *Qp = q, *Kp = k;
        if (theta) {
            FwdArgs A;
            fill_fwd(A, q, k, v, nullptr, B, N, H, dk, dv, out_dt, gamma, theta, pos0);
            A.qr = ws + L.qp;
            A.kr = ws + L.kp;
            Qp = A.qr;
            Kp = A.kr;
            LaunchTimer tr("ret_rotate_qk", s);
            hipLaunchKernelGGL(rotate_qk_get(), dim3(rotate_qk_blocks(B, N, H, dk)), dim3(256), 0, s, A);
            tr.done();
            if ((st = launch_status("ret_rotate_qk")) != RET_OK) return st;
        }
        // dq and dk straight from the retentions, their output rows turned back by the transpose rotation
        void* chain = ws + L.chain;
        if ((st = chunkwise_run(dout, v, Kp, dq, B, N, H, dv, dk, RET_BF16, out_dt, gamma, nullptr, pos0, chunk,
                                nullptr, nullptr, chain, L.chain_bytes, stream, nullptr, nullptr, false, theta)) !=
            RET_OK)
            return st;
        if ((st = chunkwise_run(Kp, Qp, dout, dv_out, B, N, H, dk, dv, RET_BF16, out_dt, gamma, nullptr, 0, chunk,
                                nullptr, nullptr, chain, L.chain_bytes, stream, nullptr, nullptr, true)) != RET_OK)
            return st;
        return chunkwise_run(v, dout, Qp, dk_out, B, N, H, dv, dk, RET_BF16, out_dt, gamma, nullptr, pos0, chunk,
                             nullptr, nullptr, chain, L.chain_bytes, stream, nullptr, nullptr, true, theta);
    }
    const int ib = in_dt == RET_BF16;
    if (L.nb == 2) {
        // dq' = sum over the two d_v halves b of retention(dO_b, V_b, K'); dk'^rev likewise of
        // retention(V_b^rev, dO_b^rev, Q'^rev); dv^rev = retention(K'^rev, Q'^rev, dO^rev) over the whole d_v
        void *Kp = ws + L.kp, *Kr = ws + L.kr, *Qr = ws + L.qr, *dOr = ws + L.dor, *chain = ws + L.chain;
        const int wb = L.wb;
        const PermJob pre[3] = {
            {k, {Kp, Kr}, dk, 1, 0, {0, 1}, ib, ib},
            {q, {Qr, nullptr}, dk, 1, 0, {1, 0}, ib, ib},
            {dout, {dOr, nullptr}, dv, 0, 0, {1, 0}, ib, ib},
        };
        if ((st = permute(pre, 3, B, N, H, theta, pos0, s)) != RET_OK) return st;
        const PermJob halves[4] = {
            {v, {ws + L.vbn[0], ws + L.vbr[0]}, wb, 0, 0, {0, 1}, ib, ib, nullptr, dv, 0},
            {v, {ws + L.vbn[1], ws + L.vbr[1]}, wb, 0, 0, {0, 1}, ib, ib, nullptr, dv, wb},
            {dout, {ws + L.dobn[0], ws + L.dobr[0]}, wb, 0, 0, {0, 1}, ib, ib, nullptr, dv, 0},
            {dout, {ws + L.dobn[1], ws + L.dobr[1]}, wb, 0, 0, {0, 1}, ib, ib, nullptr, dv, wb},
        };
        if ((st = permute(halves, 4, B, N, H, nullptr, 0, s)) != RET_OK) return st;
        for (int i = 0; i < 2; ++i)
            if ((st = chunkwise_run(ws + L.dobn[i], ws + L.vbn[i], Kp, ws + L.g1b[i], B, N, H, wb, dk, in_dt, RET_F32,
                                    gamma, nullptr, 0, chunk, nullptr, nullptr, chain, L.chain_bytes, stream, nullptr,
                                    nullptr)) != RET_OK)
                return st;
        if ((st = chain_meta_zero(in_dt, B, N, H, dk, dv, chunk, chain, L.chain_bytes, s)) != RET_OK) return st;
        if ((st = chunkwise_run(Kr, Qr, dOr, ws + L.g2, B, N, H, dk, dv, in_dt, RET_F32, gamma, nullptr, 0, chunk,
                                nullptr, nullptr, chain, L.chain_bytes, stream, nullptr, nullptr)) != RET_OK)
            return st;
        if ((st = chain_meta_zero(in_dt, B, N, H, wb, dk, chunk, chain, L.chain_bytes, s)) != RET_OK) return st;
        for (int i = 0; i < 2; ++i)
            if ((st = chunkwise_run(ws + L.vbr[i], ws + L.dobr[i], Qr, ws + L.g3b[i], B, N, H, wb, dk, in_dt, RET_F32,
                                    gamma, nullptr, 0, chunk, nullptr, nullptr, chain, L.chain_bytes, stream, nullptr,
                                    nullptr)) != RET_OK)
                return st;
        const PermJob post[3] = {
            {ws + L.g1b[0], {dq, nullptr}, dk, -1, 0, {0, 0}, 0, ob, ws + L.g1b[1]},
            {ws + L.g3b[0], {dk_out, nullptr}, dk, -1, 1, {0, 0}, 0, ob, ws + L.g3b[1]},
            {ws + L.g2, {dv_out, nullptr}, dv, 0, 1, {0, 0}, 0, ob},
        };
        return permute(post, 3, B, N, H, theta, pos0, s);
    }
    void *Kp = ws + L.kp, *Kr = ws + L.kr, *Qr = ws + L.qr, *Vr = ws + L.vr, *dOr = ws + L.dor;
    void *G1 = ws + L.g1, *G2 = ws + L.g2, *G3 = ws + L.g3, *chain = ws + L.chain;
    // inputs of the three retentions: K' in order; K', Q', V and dO reversed (one launch, in the input dtype)
    const PermJob pre[4] = {
        {k, {Kp, Kr}, dk, 1, 0, {0, 1}, ib, ib},
        {q, {Qr, nullptr}, dk, 1, 0, {1, 0}, ib, ib},
        {v, {Vr, nullptr}, dv, 0, 0, {1, 0}, ib, ib},
        {dout, {dOr, nullptr}, dv, 0, 0, {1, 0}, ib, ib},
    };
    if ((st = permute(pre, 4, B, N, H, theta, pos0, s)) != RET_OK) return st;
    // dq' = retention(dO, V, K'); dv^rev = retention(K'^rev, Q'^rev, dO^rev); dk'^rev = retention(V^rev, dO^rev, Q'^rev)
    if ((st = chunkwise_run(dout, v, Kp, G1, B, N, H, dv, dk, in_dt, RET_F32, gamma, nullptr, 0, chunk, nullptr,
                            nullptr, chain, L.chain_bytes, stream, nullptr, nullptr)) != RET_OK)
        return st;
    if (dk != dv && (st = chain_meta_zero(in_dt, B, N, H, dk, dv, chunk, chain, L.chain_bytes, s)) != RET_OK)
        return st;
    if ((st = chunkwise_run(Kr, Qr, dOr, G2, B, N, H, dk, dv, in_dt, RET_F32, gamma, nullptr, 0, chunk, nullptr,
                            nullptr, chain, L.chain_bytes, stream, nullptr, nullptr)) != RET_OK)
        return st;
    if (dk != dv && (st = chain_meta_zero(in_dt, B, N, H, dv, dk, chunk, chain, L.chain_bytes, s)) != RET_OK)
        return st;
    if ((st = chunkwise_run(Vr, dOr, Qr, G3, B, N, H, dv, dk, in_dt, RET_F32, gamma, nullptr, 0, chunk, nullptr,
                            nullptr, chain, L.chain_bytes, stream, nullptr, nullptr)) != RET_OK)
        return st;
    // back to the caller's order, dq and dk turned back by the transpose rotation
    const PermJob post[3] = {
        {G1, {dq, nullptr}, dk, -1, 0, {0, 0}, 0, ob},
        {G3, {dk_out, nullptr}, dk, -1, 1, {0, 0}, 0, ob},
        {G2, {dv_out, nullptr}, dv, 0, 1, {0, 0}, 0, ob},
    };
    return permute(post, 3, B, N, H, theta, pos0, s);
}

int ret_timing_enable(int on) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    int prev = g_timing_on;
    g_timing_on = on != 0;
    return prev;
}

int ret_timing_query(const char* kernel, double* total_ms, int64_t* launches) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    double tot = 0.0;
    int64_t n = 0;
    for (auto& r : g_timing) {
        if (kernel && *kernel && strcmp(kernel, r.name) != 0) continue;
        if (hipEventSynchronize(r.stop) != hipSuccess) return RET_ERR_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return RET_ERR_HIP;
        tot += ms;
        ++n;
    }
    if (total_ms) *total_ms = tot;
    if (launches) *launches = n;
    return RET_OK;
}

ret_status_t ret_chunkwise_check(const void* workspace, void* stream) {
    if (!workspace) return RET_OK;
    ChainHeader h;
    if (hipMemcpyAsync(&h, workspace, sizeof(h), hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess ||
        hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
        return fail(RET_ERR_HIP, "reading the workspace header failed");
    if (h.error) return fail(RET_ERR_HIP, "a segment-chain wait gave up: outputs of that call are invalid");
    return RET_OK;
}

void ret_timing_reset(void) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    for (auto& r : g_timing) {
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    g_timing.clear();
}

}  // extern "C"
