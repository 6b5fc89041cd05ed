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
#include <new>
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

}  // namespace

// ---- launch records: a caller-owned object (ret_options_t.timer); the library keeps none of its own ----
struct ret_timer {
    struct Rec {
        const char* name;
        hipEvent_t start, stop;
    };
    std::mutex mu;
    std::vector<Rec> recs;
};

namespace {

// The plan options with the library's defaults filled in (ret_options_t documents each field).
struct Opts {
    int segments = 0, target_wgs = 0, prerotate = -1, onchip = 1, variant = 0;
    int step_cw = 0, step_wr = 0, step_pairs = 0, bwd_direct = 1, step_cache = 0;
    long long chain_spin = 0;
    ret_timer_t* timer = nullptr;
};
Opts resolve(const ret_options_t* o) {
    Opts r;
    if (!o) return r;
    r.segments = o->segments > 0 ? o->segments : 0;
    r.target_wgs = o->target_wgs > 0 ? o->target_wgs : 0;
    r.prerotate = o->prerotate < 0 ? -1 : (o->prerotate != 0);
    r.onchip = o->onchip != 0;
    r.variant = o->variant;
    r.step_cw = o->step_cw;
    r.step_wr = o->step_wr;
    r.step_pairs = o->step_pairs;
    r.bwd_direct = o->bwd_direct != 0;
    r.step_cache = o->step_cache != 0;
    r.chain_spin = o->chain_spin;
    r.timer = o->timer;
    return r;
}
const Opts kDefaultOpts;

// Kernel-argument form of the chain's wait limit: ticks, or -1 (every wait gives up at once).
long long chain_spin_arg(const Opts& op) {
    if (op.chain_spin < 0) return -1;
    return op.chain_spin > 0 ? op.chain_spin : (1ll << 24);
}

struct LaunchTimer {
    hipEvent_t start = nullptr, stop = nullptr;
    hipStream_t stream;
    const char* name;
    ret_timer_t* t;
    LaunchTimer(const char* n, hipStream_t s, const Opts& op) : stream(s), name(n), t(op.timer) {
        if (t && hipEventCreate(&start) == hipSuccess && hipEventCreate(&stop) == hipSuccess)
            (void)hipEventRecord(start, stream);
        else
            t = nullptr;
    }
    void done() {
        if (!t) return;
        (void)hipEventRecord(stop, stream);
        std::lock_guard<std::mutex> lk(t->mu);
        t->recs.push_back({name, start, stop});
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
bool pick_chunk(ret_dtype_t in_dt, int dk, int dv, int C, ChunkKernels* out, const Opts& op = kDefaultOpts) {
    if (in_dt == RET_F32) return chunk_kernels_f32(dk, dv, C, out);
    if (dk == 32 || dk == 64) return chunk_kernels_bf16_small(dk, dv, C, out);
    if (dk == 128) return chunk_kernels_bf16_128(dk, dv, C, op.variant, out);
    if (dk == 256) return chunk_kernels_bf16_256(dk, dv, C, op.variant, out);
    return false;
}

bool pick_parallel(ret_dtype_t in_dt, int dk, int dv, ParKernel* out) {
    return parallel_kernel_get(in_dt == RET_BF16, dk, dv, out);
}

// ---- segment heuristic ----
// Number of segments per sequence and tokens per segment. Enough workgroups to fill the chip, but segments of
// at least ~256 tokens so the per-segment state traffic stays small against the segment's own data.
void plan_segments(int B, int N, int H, int dv, int C, int dvt, int target_wgs, const Opts& op, int* nseg,
                   int* seg_len) {
    const long long units = (long long)B * H * ((dv + dvt - 1) / dvt);
    const int nchunks = (N + C - 1) / C;
    const int target = op.target_wgs > 0 ? op.target_wgs : target_wgs > 0 ? target_wgs : 1024;
    int g = (int)((target + units - 1) / units);
    const int forced = op.segments;
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
    // the split launches: a state slot per (unit, segment) after the chain's (untouched) first kChainMeta bytes
    if (ck.split_local || ck.fused_split)
        return kChainMeta + (size_t)B * H * (dv / ck.dvt) * nseg * dk * ck.dvt * sizeof(float);
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
                     size_t avail, const Opts& op = kDefaultOpts) {
    ChunkPlan p;
    plan_segments(B, N, H, dv, chunk, ck.dvt, ck.target_wgs, op, &p.nseg, &p.seg_len);
    p.chain_bytes = (segment_ws_bytes(ck, B, H, dk, dv, p.nseg) + 255) / 256 * 256;
    p.rot_bytes = 0;
    // prerotate 0 / 1 turns the up-front rotation off / on wherever a kernel supports it.
    const int pre = op.prerotate;
    if (ck.fused_pre && rotate && (pre < 0 ? (ck.pre_always || dv / ck.dvt >= 4) : pre != 0))
        p.rot_bytes = 2 * (((size_t)B * N * H * dk * 2 + 255) / 256 * 256);
    // The rotated copies follow the chain's header, counters and flags (the first kChainMeta bytes) even when
    // the plan has no chain, so that those stay zero for any later call that shares the workspace.
    auto chain_part = [&](size_t chain) { return p.rot_bytes > 0 && chain < kChainMeta ? kChainMeta : chain; };
    if (chain_part(p.chain_bytes) + p.rot_bytes > avail) p.rot_bytes = 0;
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
    p.chain_bytes = chain_part(p.chain_bytes);
    return p;
}

// Whether a plan runs the on-chip segment kernel: chained segments short enough to stay on chip (onchip = 0
// turns it off).
bool plan_onchip(const ChunkKernels& ck, const ChunkPlan& p, const Opts& op = kDefaultOpts) {
    return ck.fused && p.nseg > 1 && ck.seg && p.seg_len <= ck.seg_tokens && op.onchip != 0;
}

}  // namespace

// =====================================================================================================
// Exported C ABI
// =====================================================================================================
extern "C" {

int ret_abi_version(void) { return RET_ABI_VERSION; }

#ifndef RET_SOURCE_DIGEST
#define RET_SOURCE_DIGEST "unknown"
#endif
const char* ret_source_digest(void) { return RET_SOURCE_DIGEST; }

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
    LaunchTimer tm("ret_parallel", s, kDefaultOpts);
    hipLaunchKernelGGL(pk.fn, grid, dim3(kThreads), 0, s, A);
    tm.done();
    return launch_status("ret_parallel");
}

size_t ret_chunkwise_workspace_bytes_ex(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt,
                                        const ret_options_t* opts) {
    const Opts op = resolve(opts);
    ChunkKernels ck;
    if (B <= 0 || N <= 0 || H <= 0 || dk <= 0 || dv <= 0 || chunk <= 0) return 0;
    if (!pick_chunk(in_dt, dk, dv, chunk, &ck, op)) return 0;
    const ChunkPlan p = plan_chunk(ck, B, N, H, dk, dv, chunk, true, SIZE_MAX, op);
    return p.chain_bytes + p.rot_bytes;
}

size_t ret_chunkwise_workspace_bytes(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt) {
    return ret_chunkwise_workspace_bytes_ex(B, N, H, dk, dv, chunk, in_dt, nullptr);
}

}  // extern "C"

namespace {

// ret_msr_epilogue's work.
ret_status_t epilogue_run(const void* o, const void* gate, const float* gn_weight, const float* gn_bias, void* y,
                          int64_t rows, int H, int dv, ret_dtype_t o_dt, ret_dtype_t gate_dt, ret_dtype_t y_dt,
                          float eps, void* stream, const Opts& op) {
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
    LaunchTimer tm("ret_msr_epilogue", s, op);
    hipLaunchKernelGGL(fn, dim3((unsigned)wgs), dim3(256), 0, s, A);
    tm.done();
    return launch_status("ret_msr_epilogue");
}

// The epilogue a chunkwise call may fuse into its output stores.
struct EpiRequest {
    const void* gate;
    ret_dtype_t gate_dt;
    const float *weight, *bias;
    float eps;
};

// ret_chunkwise_fwd's work. With `epi`, the kernel applies the epilogue to the outputs before storing them where
// it holds whole head rows (the on-chip kernel with bf16 output and d_v = 64), and *fused says whether it did.
// The kernel set and plan of a chunkwise call. A set whose kernels stage operands as given only (pre_only)
// gives way to its fallback variant when q and k need rotating and the workspace holds no rotated copies.
bool resolve_chunk(ret_dtype_t in_dt, int B, int N, int H, int dk, int dv, int chunk, bool rotate, size_t avail,
                   const Opts& op, ChunkKernels* ck, ChunkPlan* plan) {
    if (!pick_chunk(in_dt, dk, dv, chunk, ck, op)) return false;
    *plan = plan_chunk(*ck, B, N, H, dk, dv, chunk, rotate, avail, op);
    if (ck->pre_only && rotate && plan->rot_bytes == 0) {
        Opts o2 = op;
        o2.variant = ck->fallback_variant;
        if (!pick_chunk(in_dt, dk, dv, chunk, ck, o2) || ck->pre_only) return false;
        *plan = plan_chunk(*ck, B, N, H, dk, dv, chunk, rotate, avail, o2);
    }
    return true;
}

ret_status_t chunkwise_run(const void* q, const void* k, const void* v, void* o, int B, int N, int H, int dk,
                           int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma, const double* theta,
                           int64_t pos0, int chunk, const float* state_in, float* state_out, void* workspace,
                           size_t workspace_bytes, void* stream, const EpiRequest* epi, bool* fused,
                           const Opts& op, bool rev = false, const double* out_theta = nullptr, int qk_din = 0,
                           int qk_col0 = 0, bool v_rot = false, const float* states_t = nullptr) {
    if (fused) *fused = false;
    ret_status_t st = check_common(q, k, v, o, B, N, H, dk, dv, in_dt, out_dt, gamma, theta);
    if (st != RET_OK) return st;
    if (chunk <= 0) return fail(RET_ERR_INVALID_ARG, "chunk must be positive (got %d)", chunk);
    if ((state_in && !aligned16(state_in)) || (state_out && !aligned16(state_out)))
        return fail(RET_ERR_INVALID_ARG, "state buffers must be 16-byte aligned");
    if (workspace_bytes > 0 && !workspace) return fail(RET_ERR_WORKSPACE, "workspace_bytes > 0 with a null workspace");
    if (workspace && !aligned16(workspace)) return fail(RET_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    // q and k as columns qk_col0 .. qk_col0 + d_k - 1 of heads qk_din wide (16-byte aligned rows)
    if (qk_din && (qk_din % 8 || qk_col0 % 8 || qk_col0 < 0 || qk_col0 + dk > qk_din))
        return fail(RET_ERR_INVALID_ARG, "q/k column block %d..%d of heads %d wide", qk_col0, qk_col0 + dk, qk_din);
    // The kernels address one chunk of one head with 32-bit byte offsets.
    const int dmax = qk_din > dk ? qk_din : dk;
    if ((long long)chunk * H * (dmax > dv ? dmax : dv) * 4 >= (1LL << 31))
        return fail(RET_ERR_UNSUPPORTED, "chunkwise form: chunk*H*max(d_k,d_v) too large (%d*%d*%d)", chunk, H,
                    dk > dv ? dk : dv);
    ChunkKernels ck;
    ChunkPlan plan;
    if (!resolve_chunk(in_dt, B, N, H, dk, dv, chunk, theta != nullptr, workspace_bytes, op, &ck, &plan))
        return fail(RET_ERR_UNSUPPORTED, "chunkwise form: unsupported d_k=%d d_v=%d chunk=%d for %s input", dk, dv,
                    chunk, in_dt == RET_F32 ? "F32" : "BF16");
    if (rev && !ck.fused) return fail(RET_ERR_UNSUPPORTED, "reversed chunkwise run: not available for this shape");
    const int nseg = plan.nseg, seg_len = plan.seg_len;

    FwdArgs A;
    fill_fwd(A, q, k, v, o, B, N, H, dk, dv, out_dt, gamma, theta, pos0);
    A.state_in = state_in;
    A.state_out = state_out;
    // The split kernels keep their segment states after the (unused, zero) chain header.
    A.ws = ck.fused || !workspace ? (float*)workspace : (float*)((char*)workspace + sizeof(ChainHeader));
    A.nseg = nseg;
    A.seg_len = seg_len;
    A.chain_spin = chain_spin_arg(op);
    hipStream_t s = (hipStream_t)stream;
    const int ntiles = dv / ck.dvt;
    if (ck.fused) {
        // Segments short enough to stay on chip take the on-chip variant.
        const bool onchip = plan_onchip(ck, plan, op);
        // Staging copies rows instead of rotating them when there is no rotation, or when q and k are rotated
        // once up front (several d_v tiles stage the same rows).
        // (reversed runs with rotation: the reversed instance that rotates q and k while staging)
        const bool rot_rev = rev && theta && plan.rot_bytes == 0 && !qk_din && !out_theta && !v_rot &&
                             (onchip ? ck.seg_rot_rev != nullptr : ck.fused_rot_rev && N % ck.rev_step == 0);
        fwd_kernel_t fn = rot_rev ? (onchip ? ck.seg_rot_rev : ck.fused_rot_rev) : onchip ? ck.seg : ck.fused;
        const fwd_kernel_t fn_pre = onchip ? (rev ? ck.seg_rev : ck.seg_pre)
                                           : (rev && !ck.split_local ? ck.fused_rev : ck.fused_pre);
        // The reversed run and the rotation of the outputs exist for the on-chip kernel, the reversed run and q, k
        // taken from wider heads for the three-launch kernels, and the reversed run and (chunk_fused_bf16) the
        // rotation of the outputs for the single-pass kernels that have them (whole steps only when reversed); all
        // without input rotation, state or epilogue.
        if (rev || out_theta || qk_din || v_rot) {
            const bool plain = (!theta || rot_rev) && !state_in && !state_out && !epi;
            const bool seg_ok = onchip && !qk_din && (!rev || ck.seg_rev) && (!v_rot || out_theta);
            const bool split_ok = ck.split_local && !onchip && !out_theta && (!rev || N % kDmaStep == 0);
            const bool fused_ok = !ck.split_local && !onchip && !qk_din &&
                                  (!rev || (ck.fused_rev && N % ck.rev_step == 0)) &&
                                  (!(out_theta || v_rot) || ck.fused_orot) && (!v_rot || out_theta);
            if (!plain || !(seg_ok || split_ok || fused_ok))
                return fail(RET_ERR_UNSUPPORTED, "reversed, output-rotated or column-block chunkwise run: not "
                                                 "available for this shape");
        }
        if (states_t && ck.split_local)
            return fail(RET_ERR_UNSUPPORTED, "chunkwise form: transposed entering states with this plan");
        if (out_theta) {
            A.orot = 1;
            A.vrot = v_rot;  // (v has the outputs' width: one rotation for both)
            for (int i = 0; i < dv / 2; ++i) A.theta[i] = out_theta[i];
        }
        if (!theta) {
            fn = fn_pre;
            A.qr = const_cast<void*>(q);
            A.kr = const_cast<void*>(k);
        } else if (plan.rot_bytes > 0) {
            fn = fn_pre;
            A.qr = (char*)workspace + plan.chain_bytes;
            A.kr = (char*)A.qr + plan.rot_bytes / 2;
            LaunchTimer tr("ret_rotate_qk", s, op);
            hipLaunchKernelGGL(rotate_qk_get(), dim3(rotate_qk_blocks(B, N, H, dk)), dim3(256), 0, s, A);
            tr.done();
            if ((st = launch_status("ret_rotate_qk")) != RET_OK) return st;
        }
        const unsigned grid = (unsigned)((long long)nseg * B * H * ntiles);
        if (ck.pre_only && fn != fn_pre)
            return fail(RET_ERR_UNSUPPORTED, "chunkwise form: kernel set without in-staging rotation");
        if (ck.split_local) {
            // local passes, the scan of their states, then the full pass of every segment (no chain)
            if (epi || onchip) return fail(RET_ERR_UNSUPPORTED, "chunkwise form: split launches with this plan");
            A.ws = workspace ? (float*)((char*)workspace + kChainMeta) : nullptr;
            A.qk_din = qk_din;
            A.qk_col0 = qk_col0;
            const unsigned units = (unsigned)((long long)B * H * ntiles);
            if (rev && (!ck.split_local_rev || !ck.split_full_rev))
                return fail(RET_ERR_UNSUPPORTED, "reversed chunkwise run: not available for this shape");
            if (nseg > 1) {
                LaunchTimer tl("ret_chunk_dma_local", s, op);
                hipLaunchKernelGGL(rev ? ck.split_local_rev : ck.split_local, dim3(units * (unsigned)(nseg - 1)),
                                   dim3(ck.threads_pre), 0, s, A);
                tl.done();
                if ((st = launch_status("ret_chunk_dma_local")) != RET_OK) return st;
                LaunchTimer tc("ret_chunk_dma_scan", s, op);
                hipLaunchKernelGGL(ck.split_scan, dim3((unsigned)((long long)dk * ck.dvt / 1024), units), dim3(256), 0,
                                   s, A);
                tc.done();
                if ((st = launch_status("ret_chunk_dma_scan")) != RET_OK) return st;
            }
            LaunchTimer tm(ck.pre_name, s, op);
            hipLaunchKernelGGL(rev ? ck.split_full_rev : fn, dim3(grid), dim3(ck.threads_pre), 0, s, A);
            tm.done();
            return launch_status(ck.pre_name);
        }
        const bool pre = !onchip && (fn == ck.fused_pre || (rev && fn == ck.fused_rev));
        const int threads = onchip || !ck.threads ? kThreads : pre && ck.threads_pre ? ck.threads_pre : ck.threads;
        const char* name = onchip ? "ret_chunk_seg" : pre && ck.pre_name ? ck.pre_name : "ret_chunk_fused";
        if (states_t && !(ck.fused_split && ck.fused_orot && pre && nseg > 1 && dk == dv && dv == ck.dvt && !epi))
            return fail(RET_ERR_UNSUPPORTED, "chunkwise form: transposed entering states with this plan");
        if (ck.fused_split && !onchip && nseg > 1 && !epi) {
            // local passes, the scan of their states, then the full pass of every segment (no chain); or, given
            // the states of another run (states_t), the full passes alone, entering with their transposes
            A.ws = workspace ? (float*)((char*)workspace + kChainMeta) : nullptr;
            const unsigned units = (unsigned)((long long)B * H * ntiles);
            if (states_t) {
                A.ws_t = states_t;
            } else {
                A.split = 1;
                LaunchTimer tl("ret_chunk_fused_local", s, op);
                hipLaunchKernelGGL(fn, dim3(units * (unsigned)(nseg - 1)), dim3(threads), 0, s, A);
                tl.done();
                if ((st = launch_status("ret_chunk_fused_local")) != RET_OK) return st;
                LaunchTimer tc("ret_chunk_fused_scan", s, op);
                hipLaunchKernelGGL(slot_scan_get(), dim3((unsigned)((long long)dk * ck.dvt / 512), units), dim3(256),
                                   0, s, A);
                tc.done();
                if ((st = launch_status("ret_chunk_fused_scan")) != RET_OK) return st;
            }
            A.split = 2;
            LaunchTimer tm(name, s, op);
            hipLaunchKernelGGL(fn, dim3(grid), dim3(threads), 0, s, A);
            tm.done();
            return launch_status(name);
        }
        if (epi && onchip && out_dt == RET_BF16 && dv == 64) {
            A.epi = 1;
            A.gate = epi->gate;
            A.gate_bf16 = epi->gate_dt == RET_BF16;
            A.gn_weight = epi->weight;
            A.gn_bias = epi->bias;
            A.eps = epi->eps;
            if (fused) *fused = true;
        }
        LaunchTimer tm(name, s, op);
        hipLaunchKernelGGL(fn, dim3(grid), dim3(threads), 0, s, A);
        tm.done();
        return launch_status(name);
    }
    if (nseg > 1) {
        {
            LaunchTimer tm("ret_chunk_local", s, op);
            hipLaunchKernelGGL(ck.local, dim3(nseg - 1, ntiles, B * H), dim3(kThreads), 0, s, A);
            tm.done();
            if ((st = launch_status("ret_chunk_local")) != RET_OK) return st;
        }
        {
            const long long per4 = (long long)dk * dv / 4;
            LaunchTimer tm("ret_segment_scan", s, op);
            hipLaunchKernelGGL(segment_scan_get(), dim3((unsigned)((per4 + kThreads - 1) / kThreads), B * H),
                               dim3(kThreads), 0, s, A);
            tm.done();
            if ((st = launch_status("ret_segment_scan")) != RET_OK) return st;
        }
    }
    LaunchTimer tm("ret_chunk_full", s, op);
    hipLaunchKernelGGL(ck.full, dim3(nseg, ntiles, B * H), dim3(kThreads), 0, s, A);
    tm.done();
    return launch_status("ret_chunk_full");
}

// Workspace of the gradients. At offset 0 the segment chain (or the segment states) the retentions share (one
// call after another; at least 256 bytes, so ret_chunkwise_check reads its header). Then:
// - when both reversed retentions run on the on-chip kernel's reversed traversal (direct, bf16 only): Q' and K'
//   (bf16, only with rotation);
// - when every retention runs in place over reversed rows and d_v blocks (inplace: the three-launch kernels, or
//   with one block the single-pass kernels' reversed instances; bf16, N a multiple of their step): Q' and K' (only
//   with rotation), then (room for fp32, held in the gradients' precision) the dq' of each d_v block and the dk'
//   of each block, each set contiguous; none where the streaming kernel writes dq and dk itself (own_out);
// - otherwise the reordered inputs (K', K' reversed, Q' reversed, and V and dO reversed, or their blocks forward
//   and reversed) in the input dtype, and the fp32 outputs.
struct BwdLayout {
    bool direct, inplace;
    bool own_out;    // in place with one block, on single-pass kernels that write dq and dk themselves
    bool stage_rot;  // own_out, and the kernels rotate while staging: no rotated copies of q and k
    int variant;  // kernel variant of the retentions (the wide-head kernels' where the in-place path takes them)
    int nb, wb;  // d_v blocks of width wb for the retentions that contract over d_v (nb = 2 when d_v is wider
                 // than their kernels' d_k; dq' and dk' are then sums of two retentions)
    size_t qp, kp, kr, qr, vr, dor, g1, g2, g3, chain, chain_bytes, total;
    size_t vbn[2], dobn[2], vbr[2], dobr[2], g1b[2], g3b[2];  // per block (nb = 2)
};
bool bwd_layout(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt, bool rotate, BwdLayout* L,
                const Opts& op = kDefaultOpts) {
    ChunkKernels ca, cb;
    memset(L, 0, sizeof(*L));
    L->nb = 1;
    L->wb = dv;
    if (!pick_chunk(in_dt, dv, dk, chunk, &ca, op)) {
        // d_v too wide to be the contraction width of a retention: two halves, each a retention of its own
        if (dv % 2 || (dv / 2) % 16 || !pick_chunk(in_dt, dv / 2, dk, chunk, &ca, op)) return false;
        L->nb = 2;
        L->wb = dv / 2;
    }
    if (!pick_chunk(in_dt, dk, dv, chunk, &cb, op)) return false;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t nk = (size_t)B * N * H * dk, nv = (size_t)B * N * H * dv, es = in_dt == RET_BF16 ? 2 : 4;
    const size_t nw = (size_t)B * N * H * L->wb;
    const ChunkPlan pa = plan_chunk(ca, B, N, H, L->wb, dk, chunk, false, SIZE_MAX, op);
    const ChunkPlan pb = plan_chunk(cb, B, N, H, dk, dv, chunk, false, SIZE_MAX, op);
    L->direct = in_dt == RET_BF16 && L->nb == 1 && plan_onchip(ca, pa, op) && ca.seg_rev && plan_onchip(cb, pb, op) &&
                cb.seg_rev && op.bwd_direct != 0;
    // (direct: the dq' and dk' runs turn their v rows while staging, the dv run rotates its q and k while staging)
    if (L->direct) L->stage_rot = rotate && cb.seg_rot_rev;
    L->variant = op.variant;
    L->inplace = !L->direct && in_dt == RET_BF16 && N % kDmaStep == 0 && ca.split_local &&
                 !plan_onchip(ca, pa, op) && cb.split_local && !plan_onchip(cb, pb, op) && op.bwd_direct != 0;
    L->chain = 0;
    L->chain_bytes = pa.chain_bytes > pb.chain_bytes ? pa.chain_bytes : pb.chain_bytes;
    // Otherwise, with one block of d_v, the single-pass kernels that have reversed instances: the shape's own set,
    // else (default variant) the wide-head kernels'.
    const int tries[2] = {op.variant, op.variant == 0 ? 3 : -1};
    for (int t = 0; t < 2 && !L->direct && !L->inplace && in_dt == RET_BF16 && L->nb == 1 && op.bwd_direct != 0; ++t) {
        if (tries[t] < 0) break;
        Opts ot = op;
        ot.variant = tries[t];
        ChunkKernels wa, wb;
        if (!pick_chunk(in_dt, L->wb, dk, chunk, &wa, ot) || !wa.fused_rev || N % wa.rev_step ||
            !pick_chunk(in_dt, dk, dv, chunk, &wb, ot) || !wb.fused_rev || N % wb.rev_step)
            continue;
        const ChunkPlan qa = plan_chunk(wa, B, N, H, L->wb, dk, chunk, false, SIZE_MAX, ot);
        const ChunkPlan qb = plan_chunk(wb, B, N, H, dk, dv, chunk, false, SIZE_MAX, ot);
        if (plan_onchip(wa, qa, ot) || plan_onchip(wb, qb, ot)) continue;
        L->inplace = true;
        L->variant = tries[t];
        L->chain_bytes = qa.chain_bytes > qb.chain_bytes ? qa.chain_bytes : qb.chain_bytes;
    }
    // With one block of d_v, retentions on the single-pass kernels write dq and dk themselves, turned back by the
    // transpose rotation in their kernels: no fp32 outputs in the workspace and no final reordering launch.
    if (L->inplace && L->nb == 1) {
        Opts ot = op;
        ot.variant = L->variant;
        ChunkKernels ko;
        L->own_out = pick_chunk(in_dt, L->wb, dk, chunk, &ko, ot) && !ko.split_local && ko.fused_rev &&
                     N % ko.rev_step == 0 && (!rotate || ko.fused_orot);
        // With rotation, the dq' and dk' runs can turn their v (K, Q) while staging, and the dv run can rotate its
        // q and k (K, Q) while staging on its reversed rotating instance: then Q', K' are never written.
        ChunkKernels kv;
        L->stage_rot = L->own_out && rotate && pick_chunk(in_dt, dk, dv, chunk, &kv, ot) && !kv.split_local &&
                       kv.fused_rot_rev && N % kv.rev_step == 0 &&
                       !plan_onchip(kv, plan_chunk(kv, B, N, H, dk, dv, chunk, false, SIZE_MAX, ot), ot);
    }
    size_t off = up(L->chain_bytes > 256 ? L->chain_bytes : 256);
    if (L->direct || L->inplace) {
        if (rotate && !L->stage_rot) {
            L->qp = off;
            L->kp = L->qp + up(nk * 2);
            off = L->kp + up(nk * 2);
        }
        if (L->inplace && !L->own_out) {  // dq' of each block, then dk' of each block (one launch may write both)
            for (int i = 0; i < L->nb; ++i, off += up(nk * 4)) L->g1b[i] = off;
            for (int i = 0; i < L->nb; ++i, off += up(nk * 4)) L->g3b[i] = off;
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
                             size_t chain_bytes, hipStream_t s, const Opts& op) {
    ChunkKernels ck;
    // the split kernels keep no flags
    if (!pick_chunk(in_dt, dk, dv, chunk, &ck, op) || !ck.fused || ck.split_local || ck.fused_split) return RET_OK;
    const ChunkPlan p = plan_chunk(ck, B, N, H, dk, dv, chunk, false, chain_bytes, op);
    if (p.nseg <= 1) return RET_OK;
    const ChainLayout lay = chain_layout(B * H * (dv / ck.dvt), p.nseg, dk * ck.dvt);
    const long long n = (long long)(lay.agg_off - lay.ctr_off) / 4;
    hipLaunchKernelGGL(zero_words_get(), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (int*)((char*)chain + lay.ctr_off), n);
    return launch_status("chain_meta_zero");
}

// One launch of permute_rotate_kernel over the given jobs (at most kMaxPermJobs), one grid row per job.
ret_status_t permute(const PermJob* jobs, int njobs, int B, int N, int H, const double* theta, int64_t pos0,
                     hipStream_t s, const Opts& op) {
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
    LaunchTimer tm("ret_permute_rotate", s, op);
    hipLaunchKernelGGL(permute_rotate_get(), dim3((unsigned)((threads + 255) / 256), njobs), dim3(256), 0, s, P);
    tm.done();
    return launch_status("ret_permute_rotate");
}

}  // namespace

extern "C" {

ret_status_t ret_chunkwise_fwd_ex(const void* q, const void* k, const void* v, void* o, int B, int N, int H, int dk,
                                  int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                                  const double* theta, int64_t pos0, int chunk, const float* state_in,
                                  float* state_out, void* workspace, size_t workspace_bytes, void* stream,
                                  const ret_options_t* opts) {
    return chunkwise_run(q, k, v, o, B, N, H, dk, dv, in_dt, out_dt, gamma, theta, pos0, chunk, state_in, state_out,
                         workspace, workspace_bytes, stream, nullptr, nullptr, resolve(opts));
}

ret_status_t ret_chunkwise_fwd(const void* q, const void* k, const void* v, void* o, int B, int N, int H, int dk,
                               int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                               const double* theta, int64_t pos0, int chunk, const float* state_in,
                               float* state_out, void* workspace, size_t workspace_bytes, void* stream) {
    return ret_chunkwise_fwd_ex(q, k, v, o, B, N, H, dk, dv, in_dt, out_dt, gamma, theta, pos0, chunk, state_in,
                                state_out, workspace, workspace_bytes, stream, nullptr);
}

ret_status_t ret_chunkwise_msr_fwd(const void* q, const void* k, const void* v, const void* gate, void* y, int B,
                                   int N, int H, int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt,
                                   ret_dtype_t gate_dt, const float* gamma, const double* theta, int64_t pos0,
                                   int chunk, const float* state_in, float* state_out, const float* gn_weight,
                                   const float* gn_bias, float eps, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    return ret_chunkwise_msr_fwd_ex(q, k, v, gate, y, B, N, H, dk, dv, in_dt, out_dt, gate_dt, gamma, theta, pos0,
                                    chunk, state_in, state_out, gn_weight, gn_bias, eps, workspace, workspace_bytes,
                                    stream, nullptr);
}

ret_status_t ret_chunkwise_msr_fwd_ex(const void* q, const void* k, const void* v, const void* gate, void* y, int B,
                                      int N, int H, int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt,
                                      ret_dtype_t gate_dt, const float* gamma, const double* theta, int64_t pos0,
                                      int chunk, const float* state_in, float* state_out, const float* gn_weight,
                                      const float* gn_bias, float eps, void* workspace, size_t workspace_bytes,
                                      void* stream, const ret_options_t* opts) {
    const Opts op = resolve(opts);
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
                                    state_out, workspace, workspace_bytes, stream, &epi, &fused, op);
    if (st != RET_OK || fused) return st;
    // not fused: the retention outputs are in y; the epilogue runs over them in place
    return epilogue_run(y, gate, gn_weight, gn_bias, y, (int64_t)B * N, H, dv, out_dt, gate_dt, out_dt, eps, stream,
                        op);
}

}  // extern "C"

namespace {

// One decode step; positions either one for the call (`pos`) or one per sequence (`pos_dev`, device [B]).
ret_status_t step_run(const void* q, const void* k, const void* v, void* o, float* state, int B, int H, int dk,
                      int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma, const double* theta,
                      int64_t pos, const int64_t* pos_dev, void* stream, const Opts& op) {
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
    step_kernel_t fn = step_kernel_get(in_dt == RET_BF16, dk, dv, B * H, op.step_cw, op.step_wr, op.step_pairs,
                                       A.pos != nullptr, !op.step_cache, &cw, &wr, &ppw);
    if (!fn) return fail(RET_ERR_UNSUPPORTED, "decode step: d_k=%d not in {16,32,64,128,256}", dk);
    hipStream_t s = (hipStream_t)stream;
    LaunchTimer tm("ret_recurrent_step", s, op);
    hipLaunchKernelGGL(fn, dim3((dv + cw - 1) / cw, (B * H + ppw - 1) / ppw), dim3(64 * (dk / wr) * ppw), 0, s, A);
    tm.done();
    return launch_status("ret_recurrent_step");
}

}  // namespace

extern "C" {

ret_status_t ret_recurrent_step_ex(const void* q, const void* k, const void* v, void* o, float* state, int B, int H,
                                   int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                                   const double* theta, int64_t pos, void* stream, const ret_options_t* opts) {
    return step_run(q, k, v, o, state, B, H, dk, dv, in_dt, out_dt, gamma, theta, pos, nullptr, stream,
                    resolve(opts));
}

ret_status_t ret_recurrent_step(const void* q, const void* k, const void* v, void* o, float* state, int B, int H,
                                int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                                const double* theta, int64_t pos, void* stream) {
    return ret_recurrent_step_ex(q, k, v, o, state, B, H, dk, dv, in_dt, out_dt, gamma, theta, pos, stream, nullptr);
}

ret_status_t ret_recurrent_step_positions_ex(const void* q, const void* k, const void* v, void* o, float* state,
                                             int B, int H, int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt,
                                             const float* gamma, const double* theta, const int64_t* pos,
                                             void* stream, const ret_options_t* opts) {
    if (!pos) return fail(RET_ERR_INVALID_ARG, "null pos");
    if ((uintptr_t)pos % 8) return fail(RET_ERR_INVALID_ARG, "pos must be 8-byte aligned");
    return step_run(q, k, v, o, state, B, H, dk, dv, in_dt, out_dt, gamma, theta, 0, pos, stream, resolve(opts));
}

ret_status_t ret_recurrent_step_positions(const void* q, const void* k, const void* v, void* o, float* state, int B,
                                          int H, int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt,
                                          const float* gamma, const double* theta, const int64_t* pos,
                                          void* stream) {
    return ret_recurrent_step_positions_ex(q, k, v, o, state, B, H, dk, dv, in_dt, out_dt, gamma, theta, pos, stream,
                                           nullptr);
}

ret_status_t ret_msr_epilogue(const void* o, const void* gate, const float* gn_weight, const float* gn_bias,
                              void* y, int64_t rows, int H, int dv, ret_dtype_t o_dt, ret_dtype_t gate_dt,
                              ret_dtype_t y_dt, float eps, void* stream) {
    return epilogue_run(o, gate, gn_weight, gn_bias, y, rows, H, dv, o_dt, gate_dt, y_dt, eps, stream, kDefaultOpts);
}

ret_status_t ret_chunkwise_bwd(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk_out,
                               void* dv_out, int B, int N, int H, int dk, int dv, ret_dtype_t in_dt,
                               ret_dtype_t out_dt, const float* gamma, const double* theta, int64_t pos0, int chunk,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return ret_chunkwise_bwd_ex(q, k, v, dout, dq, dk_out, dv_out, B, N, H, dk, dv, in_dt, out_dt, gamma, theta, pos0,
                                chunk, workspace, workspace_bytes, stream, nullptr);
}

size_t ret_chunkwise_bwd_workspace_bytes_ex(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt,
                                            const ret_options_t* opts) {
    BwdLayout L;
    if (B <= 0 || N <= 0 || H <= 0 || dk <= 0 || dv <= 0 || chunk <= 0) return 0;
    if (in_dt != RET_F32 && in_dt != RET_BF16) return 0;
    if (!bwd_layout(B, N, H, dk, dv, chunk, in_dt, true, &L, resolve(opts))) return 0;
    return L.total;
}

size_t ret_chunkwise_bwd_workspace_bytes(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt) {
    return ret_chunkwise_bwd_workspace_bytes_ex(B, N, H, dk, dv, chunk, in_dt, nullptr);
}

ret_status_t ret_chunkwise_bwd_ex(const void* q, const void* k, const void* v, const void* dout, void* dq,
                                  void* dk_out, void* dv_out, int B, int N, int H, int dk, int dv, ret_dtype_t in_dt,
                                  ret_dtype_t out_dt, const float* gamma, const double* theta, int64_t pos0,
                                  int chunk, void* workspace, size_t workspace_bytes, void* stream,
                                  const ret_options_t* opts) {
    return ret_chunkwise_bwd_saved_ex(q, k, v, dout, dq, dk_out, dv_out, B, N, H, dk, dv, in_dt, out_dt, gamma, theta,
                                      pos0, chunk, nullptr, 0, workspace, workspace_bytes, stream, opts);
}

ret_status_t ret_chunkwise_bwd_saved_ex(const void* q, const void* k, const void* v, const void* dout, void* dq,
                                        void* dk_out, void* dv_out, int B, int N, int H, int dk, int dv,
                                        ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma, const double* theta,
                                        int64_t pos0, int chunk, const void* fwd_workspace, size_t fwd_workspace_bytes,
                                        void* workspace, size_t workspace_bytes, void* stream,
                                        const ret_options_t* opts) {
    const Opts op = resolve(opts);
    if (fwd_workspace && !aligned16(fwd_workspace)) return fail(RET_ERR_INVALID_ARG, "fwd_workspace must be aligned");
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
    if (!bwd_layout(B, N, H, dk, dv, chunk, in_dt, theta != nullptr, &L, op))
        return fail(RET_ERR_UNSUPPORTED,
                    "gradients: d_k=%d d_v=%d chunk=%d for %s input (both (d_k, d_v) and (d_v, d_k) need kernels)", dk,
                    dv, chunk, in_dt == RET_F32 ? "F32" : "BF16");
    if (!workspace || workspace_bytes < L.total)
        return fail(RET_ERR_WORKSPACE, "gradients need a workspace of %zu bytes (got %zu)", L.total, workspace_bytes);
    if (!aligned16(workspace)) return fail(RET_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    const int ob = out_dt == RET_BF16;
    if (L.inplace) {
        // Q', K' (rotated once), then, with the d_v blocks b of dO and V read in place:
        //   dq' = sum over b of retention(dO_b, V_b, K')
        //   dv  = retention(K', Q', dO) over the reversed sequence, rows read and written in reverse order
        //   dk' = sum over b of retention(V_b, dO_b, Q') over the reversed sequence
        // dv is written as the output; dq and dk are the block sums turned back by the transpose rotation. The
        // retentions run on the three-launch kernels, or (one block) on single-pass kernels with reversed
        // instances, whose segment chain is cleared between calls of different shapes.
        Opts ov = op;
        ov.variant = L.variant;
        void* chain = ws + L.chain;
        const int wb = L.wb, din = L.nb > 1 ? dv : 0;
        // On the three-launch kernels with square states (d_k = d_v / blocks = 256) and several segments, dq' and
        // dk' carry the transposes of (d_k, d_v)-shaped states, block by block: dq' that of sum K'_t^T V_t (the
        // forward's), dk' that of sum Q'_t^T dO_t over the reversed sequence (the dv retention's). So one local
        // pass and scan over (K', V) give dq' its segment states, the dv retention's give dk' theirs, and dq' and
        // dk' each run as one full-pass launch over all blocks that enters each segment with the transposed state
        // (no local passes or scans of their own).
        ChunkKernels ck_sq, ck_bl;
        ChunkPlan plan_sq;
        const bool share = L.variant != 3 && wb == kDmaDvt && dk == kDmaDvt &&
                           resolve_chunk(RET_BF16, B, N, H, dk, dv, chunk, false, L.chain_bytes, ov, &ck_sq, &plan_sq) &&
                           ck_sq.split_local && plan_sq.nseg > 1 && pick_chunk(RET_BF16, wb, dk, chunk, &ck_bl, ov) &&
                           ck_bl.split_full_rev && ck_bl.dvt == dk;
        // One block on the streaming kernel's split launches with square states (d_k = d_v = its tile): dk' enters
        // its segments with the transposes of the dv retention's states, and (after the forward) dq' with those of
        // the forward's, Σ K'^T V, so neither runs local passes or a scan of its own.
        bool own_square = false;
        const float* own_fws_states = nullptr;
        if (L.own_out && dk == dv) {
            ChunkKernels ka, kb;
            ChunkPlan pla, plb;
            own_square = resolve_chunk(RET_BF16, B, N, H, wb, dk, chunk, false, L.chain_bytes, ov, &ka, &pla) &&
                         resolve_chunk(RET_BF16, B, N, H, dk, dv, chunk, false, L.chain_bytes, ov, &kb, &plb) &&
                         ka.fused_split && kb.fused_split && ka.fused_orot && ka.dvt == dk && kb.dvt == dv &&
                         !plan_onchip(ka, pla, ov) && !plan_onchip(kb, plb, ov) && pla.nseg > 1 &&
                         pla.nseg == plb.nseg && pla.seg_len == plb.seg_len;
            ChunkKernels kf;
            ChunkPlan plf;
            if (own_square && fwd_workspace &&
                resolve_chunk(RET_BF16, B, N, H, dk, dv, chunk, theta != nullptr, fwd_workspace_bytes, op, &kf, &plf) &&
                kf.fused_split && kf.dvt == dv && !plan_onchip(kf, plf, op) && plf.nseg == pla.nseg &&
                plf.seg_len == pla.seg_len)
                own_fws_states = (const float*)((const char*)fwd_workspace + kChainMeta);
        }
        // The forward's workspace holds Q', K' and those same (K', V) states when its plan (with rotation, in its
        // workspace) ran the three-launch kernels over the same segments: then they are read from there.
        const char* fws = nullptr;
        ChunkPlan plan_f;
        if (share && fwd_workspace) {
            ChunkKernels ck_f;
            if (resolve_chunk(RET_BF16, B, N, H, dk, dv, chunk, theta != nullptr, fwd_workspace_bytes, op, &ck_f,
                              &plan_f) &&
                ck_f.split_local && plan_f.nseg == plan_sq.nseg && plan_f.seg_len == plan_sq.seg_len &&
                (!theta || plan_f.rot_bytes > 0))
                fws = (const char*)fwd_workspace;
        }
        // Q', K': the forward's copies, or rotated here, or (stage_rot) q and k as given, rotated while staging
        const void *Qp = q, *Kp = k;
        if (theta && fws && !L.stage_rot) {
            Qp = fws + plan_f.chain_bytes;
            Kp = (const char*)Qp + plan_f.rot_bytes / 2;
        } else if (theta && !L.stage_rot) {
            FwdArgs A;
            fill_fwd(A, q, k, v, nullptr, B, N, H, dk, dv, out_dt, gamma, theta, pos0);
            A.qr = ws + L.qp;
            A.kr = ws + L.kp;
            Qp = A.qr;
            Kp = A.kr;
            LaunchTimer tr("ret_rotate_qk", s, op);
            hipLaunchKernelGGL(rotate_qk_get(), dim3(rotate_qk_blocks(B, N, H, dk)), dim3(256), 0, s, A);
            tr.done();
            if ((st = launch_status("ret_rotate_qk")) != RET_OK) return st;
        }
        float* const slots = (float*)((char*)chain + kChainMeta);  // segment states of the (d_k, d_v) runs
        // The blocks' dq' and dk' (summed and turned back by the last launch) are kept in the gradients' own
        // precision: bf16 for bf16 gradients, which halves what they write and the last launch reads.
        const ret_dtype_t pdt = ob ? RET_BF16 : RET_F32;
        const int psz = ob ? 2 : 4;
        // every block's dq' (rev = false) or dk' (rev = true) in one full-pass launch from the transposed states
        auto blocks_from_t = [&](const void* qq, const void* kk, const void* vv, void* out, bool rev,
                                 const float* states) {
            FwdArgs A;
            fill_fwd(A, qq, kk, vv, out, B, N, H, wb, dk, pdt, gamma, nullptr, 0);
            A.qr = const_cast<void*>(qq);
            A.kr = const_cast<void*>(kk);
            A.nseg = plan_sq.nseg;
            A.seg_len = plan_sq.seg_len;
            A.qk_din = din;
            A.qk_blocks = L.nb;
            A.o_block = L.nb > 1 ? (long long)(rev ? L.g3b[1] - L.g3b[0] : L.g1b[1] - L.g1b[0]) / psz : 0;
            A.ws_t = states;
            const unsigned grid = (unsigned)((long long)B * H * L.nb * plan_sq.nseg);
            LaunchTimer tm(ck_bl.pre_name, s, ov);
            hipLaunchKernelGGL(rev ? ck_bl.split_full_rev : ck_bl.fused_pre, dim3(grid), dim3(kDmaThreads), 0, s, A);
            tm.done();
            return launch_status(ck_bl.pre_name);
        };
        if (share && fws) {
            // the forward's segment states, as its scan left them
            if ((st = blocks_from_t(dout, v, Kp, ws + L.g1b[0], false, (const float*)(fws + kChainMeta))) != RET_OK)
                return st;
        } else if (share) {
            // the forward's segment states: local passes and scan over (K', V) alone
            FwdArgs A;
            fill_fwd(A, nullptr, Kp, v, nullptr, B, N, H, dk, dv, RET_F32, gamma, nullptr, 0);
            A.kr = const_cast<void*>(Kp);
            A.ws = slots;
            A.nseg = plan_sq.nseg;
            A.seg_len = plan_sq.seg_len;
            const unsigned units = (unsigned)((long long)B * H * (dv / ck_sq.dvt));
            LaunchTimer tl("ret_chunk_dma_local", s, ov);
            hipLaunchKernelGGL(ck_sq.split_local, dim3(units * (unsigned)(plan_sq.nseg - 1)), dim3(kDmaThreads), 0, s,
                               A);
            tl.done();
            if ((st = launch_status("ret_chunk_dma_local")) != RET_OK) return st;
            LaunchTimer tc("ret_chunk_dma_scan", s, ov);
            hipLaunchKernelGGL(ck_sq.split_scan, dim3((unsigned)((long long)dk * ck_sq.dvt / 1024), units), dim3(256), 0,
                               s, A);
            tc.done();
            if ((st = launch_status("ret_chunk_dma_scan")) != RET_OK) return st;
            if ((st = blocks_from_t(dout, v, Kp, ws + L.g1b[0], false, slots)) != RET_OK) return st;
        } else if (L.own_out) {
            if ((st = chunkwise_run(dout, v, Kp, dq, B, N, H, wb, dk, RET_BF16, out_dt, gamma, nullptr, pos0, chunk,
                                    nullptr, nullptr, chain, L.chain_bytes, stream, nullptr, nullptr, ov, false,
                                    theta, 0, 0, L.stage_rot, own_fws_states)) != RET_OK)
                return st;
        } else {
            for (int i = 0; i < L.nb; ++i)
                if ((st = chunkwise_run(dout, v, Kp, ws + L.g1b[i], B, N, H, wb, dk, RET_BF16, pdt, gamma, nullptr,
                                        0, chunk, nullptr, nullptr, chain, L.chain_bytes, stream, nullptr, nullptr, ov,
                                        false, nullptr, din, i * wb)) != RET_OK)
                    return st;
        }
        const bool reshaped = wb != dk || dk != dv;  // the (d_k, d_v) of the runs differ
        if (reshaped && (st = chain_meta_zero(in_dt, B, N, H, dk, dv, chunk, chain, L.chain_bytes, s, ov)) != RET_OK)
            return st;
        if ((st = chunkwise_run(Kp, Qp, dout, dv_out, B, N, H, dk, dv, RET_BF16, out_dt, gamma,
                                L.stage_rot ? theta : nullptr, L.stage_rot ? pos0 : 0, chunk, nullptr, nullptr, chain,
                                L.chain_bytes, stream, nullptr, nullptr, ov, true)) != RET_OK)
            return st;
        if (share) {
            if ((st = blocks_from_t(v, dout, Qp, ws + L.g3b[0], true, slots)) != RET_OK) return st;
        } else if (L.own_out) {
            if (reshaped && (st = chain_meta_zero(in_dt, B, N, H, wb, dk, chunk, chain, L.chain_bytes, s, ov)) != RET_OK)
                return st;
            // dq and dk leave their kernels finished: nothing to reorder. With square states in split launches,
            // dk' enters its segments with the transposes of the dv retention's states, just left in the slots.
            return chunkwise_run(v, dout, Qp, dk_out, B, N, H, wb, dk, RET_BF16, out_dt, gamma, nullptr, pos0, chunk,
                                 nullptr, nullptr, chain, L.chain_bytes, stream, nullptr, nullptr, ov, true, theta, 0,
                                 0, L.stage_rot, own_square ? slots : nullptr);
        } else {
            if (reshaped && (st = chain_meta_zero(in_dt, B, N, H, wb, dk, chunk, chain, L.chain_bytes, s, ov)) != RET_OK)
                return st;
            for (int i = 0; i < L.nb; ++i)
                if ((st = chunkwise_run(v, dout, Qp, ws + L.g3b[i], B, N, H, wb, dk, RET_BF16, pdt, gamma, nullptr,
                                        0, chunk, nullptr, nullptr, chain, L.chain_bytes, stream, nullptr, nullptr, ov,
                                        true, nullptr, din, i * wb)) != RET_OK)
                    return st;
        }
        const bool two = L.nb > 1;
        const PermJob post[2] = {
            {ws + L.g1b[0], {dq, nullptr}, dk, -1, 0, {0, 0}, ob, ob, two ? ws + L.g1b[1] : nullptr},
            {ws + L.g3b[0], {dk_out, nullptr}, dk, -1, 0, {0, 0}, ob, ob, two ? ws + L.g3b[1] : nullptr},
        };
        return permute(post, 2, B, N, H, theta, pos0, s, op);
    }
    if (L.direct) {
        // Q', K' (rotated once; q and k themselves without rotation), then dq' = retention(dO, V, K') and, over
        // the reversed sequence on the reversed traversal, dv = retention(K', Q', dO) and dk' = retention(V, dO,
        // Q'), written in token order; dq' and dk' leave their kernels turned back by the transpose rotation. With
        // stage_rot no copies: the dq' and dk' runs turn their v rows (K, Q) while staging, and the dv run rotates
        // its q and k (K, Q) while staging.
        const void *Qp = q, *Kp = k;
        const bool vr = theta && L.stage_rot;
        if (theta && !L.stage_rot) {
            FwdArgs A;
            fill_fwd(A, q, k, v, nullptr, B, N, H, dk, dv, out_dt, gamma, theta, pos0);
            A.qr = ws + L.qp;
            A.kr = ws + L.kp;
            Qp = A.qr;
            Kp = A.kr;
            LaunchTimer tr("ret_rotate_qk", s, op);
            hipLaunchKernelGGL(rotate_qk_get(), dim3(rotate_qk_blocks(B, N, H, dk)), dim3(256), 0, s, A);
            tr.done();
            if ((st = launch_status("ret_rotate_qk")) != RET_OK) return st;
        }
        // dq and dk straight from the retentions, their output rows turned back by the transpose rotation
        void* chain = ws + L.chain;
        if ((st = chunkwise_run(dout, v, Kp, dq, B, N, H, dv, dk, RET_BF16, out_dt, gamma, nullptr, pos0, chunk,
                                nullptr, nullptr, chain, L.chain_bytes, stream, nullptr, nullptr, op, false, theta, 0, 0,
                                vr)) != RET_OK)
            return st;
        if ((st = chunkwise_run(Kp, Qp, dout, dv_out, B, N, H, dk, dv, RET_BF16, out_dt, gamma, vr ? theta : nullptr,
                                vr ? pos0 : 0, chunk, nullptr, nullptr, chain, L.chain_bytes, stream, nullptr, nullptr,
                                op, true)) != RET_OK)
            return st;
        return chunkwise_run(v, dout, Qp, dk_out, B, N, H, dv, dk, RET_BF16, out_dt, gamma, nullptr, pos0, chunk,
                             nullptr, nullptr, chain, L.chain_bytes, stream, nullptr, nullptr, op, true, theta, 0, 0,
                             vr);
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
        if ((st = permute(pre, 3, B, N, H, theta, pos0, s, op)) != RET_OK) return st;
        const PermJob halves[4] = {
            {v, {ws + L.vbn[0], ws + L.vbr[0]}, wb, 0, 0, {0, 1}, ib, ib, nullptr, dv, 0},
            {v, {ws + L.vbn[1], ws + L.vbr[1]}, wb, 0, 0, {0, 1}, ib, ib, nullptr, dv, wb},
            {dout, {ws + L.dobn[0], ws + L.dobr[0]}, wb, 0, 0, {0, 1}, ib, ib, nullptr, dv, 0},
            {dout, {ws + L.dobn[1], ws + L.dobr[1]}, wb, 0, 0, {0, 1}, ib, ib, nullptr, dv, wb},
        };
        if ((st = permute(halves, 4, B, N, H, nullptr, 0, s, op)) != RET_OK) return st;
        for (int i = 0; i < 2; ++i)
            if ((st = chunkwise_run(ws + L.dobn[i], ws + L.vbn[i], Kp, ws + L.g1b[i], B, N, H, wb, dk, in_dt, RET_F32,
                                    gamma, nullptr, 0, chunk, nullptr, nullptr, chain, L.chain_bytes, stream, nullptr,
                                    nullptr, op)) != RET_OK)
                return st;
        if ((st = chain_meta_zero(in_dt, B, N, H, dk, dv, chunk, chain, L.chain_bytes, s, op)) != RET_OK) return st;
        if ((st = chunkwise_run(Kr, Qr, dOr, ws + L.g2, B, N, H, dk, dv, in_dt, RET_F32, gamma, nullptr, 0, chunk,
                                nullptr, nullptr, chain, L.chain_bytes, stream, nullptr, nullptr, op)) != RET_OK)
            return st;
        if ((st = chain_meta_zero(in_dt, B, N, H, wb, dk, chunk, chain, L.chain_bytes, s, op)) != RET_OK) return st;
        for (int i = 0; i < 2; ++i)
            if ((st = chunkwise_run(ws + L.vbr[i], ws + L.dobr[i], Qr, ws + L.g3b[i], B, N, H, wb, dk, in_dt, RET_F32,
                                    gamma, nullptr, 0, chunk, nullptr, nullptr, chain, L.chain_bytes, stream, nullptr,
                                    nullptr, op)) != RET_OK)
                return st;
        const PermJob post[3] = {
            {ws + L.g1b[0], {dq, nullptr}, dk, -1, 0, {0, 0}, 0, ob, ws + L.g1b[1]},
            {ws + L.g3b[0], {dk_out, nullptr}, dk, -1, 1, {0, 0}, 0, ob, ws + L.g3b[1]},
            {ws + L.g2, {dv_out, nullptr}, dv, 0, 1, {0, 0}, 0, ob},
        };
        return permute(post, 3, B, N, H, theta, pos0, s, op);
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
    if ((st = permute(pre, 4, B, N, H, theta, pos0, s, op)) != RET_OK) return st;
    // dq' = retention(dO, V, K'); dv^rev = retention(K'^rev, Q'^rev, dO^rev); dk'^rev = retention(V^rev, dO^rev, Q'^rev)
    if ((st = chunkwise_run(dout, v, Kp, G1, B, N, H, dv, dk, in_dt, RET_F32, gamma, nullptr, 0, chunk, nullptr,
                            nullptr, chain, L.chain_bytes, stream, nullptr, nullptr, op)) != RET_OK)
        return st;
    if (dk != dv && (st = chain_meta_zero(in_dt, B, N, H, dk, dv, chunk, chain, L.chain_bytes, s, op)) != RET_OK)
        return st;
    if ((st = chunkwise_run(Kr, Qr, dOr, G2, B, N, H, dk, dv, in_dt, RET_F32, gamma, nullptr, 0, chunk, nullptr,
                            nullptr, chain, L.chain_bytes, stream, nullptr, nullptr, op)) != RET_OK)
        return st;
    if (dk != dv && (st = chain_meta_zero(in_dt, B, N, H, dv, dk, chunk, chain, L.chain_bytes, s, op)) != RET_OK)
        return st;
    if ((st = chunkwise_run(Vr, dOr, Qr, G3, B, N, H, dv, dk, in_dt, RET_F32, gamma, nullptr, 0, chunk, nullptr,
                            nullptr, chain, L.chain_bytes, stream, nullptr, nullptr, op)) != RET_OK)
        return st;
    // back to the caller's order, dq and dk turned back by the transpose rotation
    const PermJob post[3] = {
        {G1, {dq, nullptr}, dk, -1, 0, {0, 0}, 0, ob},
        {G3, {dk_out, nullptr}, dk, -1, 1, {0, 0}, 0, ob},
        {G2, {dv_out, nullptr}, dv, 0, 1, {0, 0}, 0, ob},
    };
    return permute(post, 3, B, N, H, theta, pos0, s, op);
}

}  // extern "C"

namespace {

// Workspace of the normalized chunkwise call: the chunkwise plan's workspace (at least the chain's metadata
// region), then the normalization's segment sums W [B*H][nseg][d_k] and row factors f [B*N*H] (fp32).
struct NormLayout {
    size_t chunk_bytes, w_off, f_off, total;
    int nseg;
};
bool norm_layout(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt, const Opts& op, NormLayout* L) {
    ChunkKernels ck;
    NormKernels nk;
    if (B <= 0 || N <= 0 || H <= 0 || dk <= 0 || dv <= 0 || chunk <= 0) return false;
    if (!pick_chunk(in_dt, dk, dv, chunk, &ck, op) || !norm_kernels_get(in_dt == RET_BF16, dk, &nk)) return false;
    const ChunkPlan p = plan_chunk(ck, B, N, H, dk, dv, chunk, true, SIZE_MAX, op);
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    L->nseg = (N + kNormSegTokens - 1) / kNormSegTokens;
    // the chain's header, counters and flags (first kChainMeta bytes) stay reserved even without a chain, so the
    // normalization's slots never cover what ret_chunkwise_check and later chained calls read
    L->chunk_bytes = up(p.chain_bytes + p.rot_bytes);
    if (L->chunk_bytes < kChainMeta) L->chunk_bytes = kChainMeta;
    L->w_off = L->chunk_bytes;
    L->f_off = L->w_off + up((size_t)B * H * L->nseg * dk * 4);
    L->total = L->f_off + up((size_t)B * N * H * 4);
    return true;
}

void fill_norm(NormArgs& A, const void* q, const void* k, void* o, int B, int N, int H, int dk, int dv,
               ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma, const double* theta, int64_t pos, int norm,
               const float* z_in, float* z_out) {
    memset(&A, 0, sizeof(A));
    A.q = q;
    A.k = k;
    A.o = o;
    A.z_in = z_in;
    A.z_out = z_out;
    A.B = B;
    A.N = N;
    A.H = H;
    A.dk = dk;
    A.dv = dv;
    A.in_bf16 = in_dt == RET_BF16;
    A.out_bf16 = out_dt == RET_BF16;
    A.norm = norm;
    A.rotate = theta != nullptr;
    A.pos0 = pos;
    for (int h = 0; h < H; ++h) {
        A.gamma[h] = gamma[h];
        A.lng[h] = log((double)gamma[h]);
    }
    if (theta)
        for (int i = 0; i < dk / 2; ++i) A.theta[i] = theta[i];
}

ret_status_t check_norm(int norm, const float* z_in, const float* z_out) {
    if (norm < 0 || norm > 7) return fail(RET_ERR_INVALID_ARG, "norm flags %d outside 0..7", norm);
    if ((z_in && !aligned16(z_in)) || (z_out && !aligned16(z_out)))
        return fail(RET_ERR_INVALID_ARG, "z buffers must be 16-byte aligned");
    return RET_OK;
}

}  // namespace

extern "C" {

size_t ret_chunkwise_normalized_workspace_bytes(int B, int N, int H, int dk, int dv, int chunk, ret_dtype_t in_dt,
                                                const ret_options_t* opts) {
    NormLayout L;
    if (!norm_layout(B, N, H, dk, dv, chunk, in_dt, resolve(opts), &L)) return 0;
    return L.total;
}

ret_status_t ret_chunkwise_normalized_fwd(const void* q, const void* k, const void* v, void* o, int B, int N, int H,
                                          int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                                          const double* theta, int64_t pos0, int chunk, int norm,
                                          const float* state_in, float* state_out, const float* z_in, float* z_out,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          const ret_options_t* opts) {
    const Opts op = resolve(opts);
    ret_status_t st = check_common(q, k, v, o, B, N, H, dk, dv, in_dt, out_dt, gamma, theta);
    if (st != RET_OK) return st;
    if ((st = check_norm(norm, z_in, z_out)) != RET_OK) return st;
    if (pos0 < 0) return fail(RET_ERR_INVALID_ARG, "normalized forms need pos0 >= 0 (got %lld)", (long long)pos0);
    if (chunk <= 0) return fail(RET_ERR_INVALID_ARG, "chunk must be positive (got %d)", chunk);
    NormLayout L;
    if (!norm_layout(B, N, H, dk, dv, chunk, in_dt, op, &L))
        return fail(RET_ERR_UNSUPPORTED, "normalized chunkwise form: unsupported d_k=%d d_v=%d chunk=%d", dk, dv,
                    chunk);
    if (!workspace || workspace_bytes < L.total)
        return fail(RET_ERR_WORKSPACE, "the normalized chunkwise form needs a workspace of %zu bytes (got %zu)",
                    L.total, workspace_bytes);
    if (!aligned16(workspace)) return fail(RET_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    NormKernels nk;
    norm_kernels_get(in_dt == RET_BF16, dk, &nk);
    // the plain chunkwise output and state
    st = chunkwise_run(q, k, v, o, B, N, H, dk, dv, in_dt, out_dt, gamma, theta, pos0, chunk, state_in, state_out,
                       workspace, L.chunk_bytes, stream, nullptr, nullptr, op);
    if (st != RET_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    NormArgs A;
    fill_norm(A, q, k, o, B, N, H, dk, dv, in_dt, out_dt, gamma, theta, pos0, norm, z_in, z_out);
    A.W = (float*)((char*)workspace + L.w_off);
    A.f = (float*)((char*)workspace + L.f_off);
    A.nseg = L.nseg;
    A.seg_len = kNormSegTokens;
    if (L.nseg > 1) {
        LaunchTimer tm("ret_norm_zseg", s, op);
        hipLaunchKernelGGL(nk.zseg, dim3(L.nseg - 1, B * H), dim3(64), 0, s, A);
        tm.done();
        if ((st = launch_status("ret_norm_zseg")) != RET_OK) return st;
    }
    {
        // the sums entering the segments: W[0] = z_in, W[g] = gamma^T W[g-1] + W[g] (the segment scan, d_v = 1)
        FwdArgs F;
        memset(&F, 0, sizeof(F));
        F.B = B;
        F.N = N;
        F.H = H;
        F.dk = dk;
        F.dv = 1;
        F.nseg = L.nseg;
        F.seg_len = kNormSegTokens;
        F.state_in = z_in;
        F.ws = A.W;
        for (int h = 0; h < H; ++h) F.log2g[h] = (float)log2((double)gamma[h]);
        LaunchTimer tm("ret_segment_scan", s, op);
        hipLaunchKernelGGL(segment_scan_get(), dim3((unsigned)((dk / 4 + kThreads - 1) / kThreads), B * H),
                           dim3(kThreads), 0, s, F);
        tm.done();
        if ((st = launch_status("ret_segment_scan")) != RET_OK) return st;
    }
    {
        LaunchTimer tm("ret_norm_rows", s, op);
        hipLaunchKernelGGL(nk.rows, dim3(L.nseg, B * H), dim3(64), 0, s, A);
        tm.done();
        if ((st = launch_status("ret_norm_rows")) != RET_OK) return st;
    }
    const long long groups = (long long)B * N * H * dv / 8;
    LaunchTimer tm("ret_norm_scale", s, op);
    hipLaunchKernelGGL(nk.scale, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, A);
    tm.done();
    return launch_status("ret_norm_scale");
}

ret_status_t ret_recurrent_step_normalized(const void* q, const void* k, const void* v, void* o, float* state,
                                           float* z, int B, int H, int dk, int dv, ret_dtype_t in_dt,
                                           ret_dtype_t out_dt, const float* gamma, const double* theta, int64_t pos,
                                           int norm, void* stream, const ret_options_t* opts) {
    const Opts op = resolve(opts);
    ret_status_t st = check_common(q, k, v, o, B, 1, H, dk, dv, in_dt, out_dt, gamma, theta);
    if (st != RET_OK) return st;
    if (!z) return fail(RET_ERR_INVALID_ARG, "null z (the normalized step carries the key sum)");
    if ((st = check_norm(norm, z, z)) != RET_OK) return st;
    if (pos < 0) return fail(RET_ERR_INVALID_ARG, "normalized forms need pos >= 0 (got %lld)", (long long)pos);
    NormKernels nk;
    if (!norm_kernels_get(in_dt == RET_BF16, dk, &nk))
        return fail(RET_ERR_UNSUPPORTED, "normalized decode step: d_k=%d", dk);
    if ((st = step_run(q, k, v, o, state, B, H, dk, dv, in_dt, out_dt, gamma, theta, pos, nullptr, stream, op)) !=
        RET_OK)
        return st;
    NormArgs A;
    fill_norm(A, q, k, o, B, 1, H, dk, dv, in_dt, out_dt, gamma, theta, pos, norm, z, z);
    if (theta)
        for (int i = 0; i < dk / 2; ++i) {
            const double ang = (double)pos * theta[i];
            A.rc[i] = (float)cos(ang);
            A.rs[i] = (float)sin(ang);
        }
    hipStream_t s = (hipStream_t)stream;
    LaunchTimer tm("ret_norm_step", s, op);
    hipLaunchKernelGGL(nk.step, dim3(B * H), dim3(64), 0, s, A);
    tm.done();
    return launch_status("ret_norm_step");
}

}  // extern "C"

// ---- the no-allocation chunkwise call: its workspace is a library-owned device array ----
// `scratch` is the array as the device code sees it. In host code its name is a host-side stand-in, not a
// device address: host code uses only the per-device address hipGetSymbolAddress returns (g_scratch[device]).
static __device__ __align__(256) unsigned char scratch[RET_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// The scratch array's address on the current device, looked up once per device (with that device current);
// the first call on a device also zeroes the chain's header, counters and flags there with a fill kernel on
// `s` (not a memset node, which a graph capture would record).
ret_status_t scratch_of_device(hipStream_t s, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(RET_ERR_HIP, "no current device (or device index >= %d)", kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(RET_ERR_HIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
        const long long n = (long long)(kChainMeta / 4);
        hipLaunchKernelGGL(zero_words_get(), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (int*)p, n);
        ret_status_t st = launch_status("scratch set-up");
        if (st != RET_OK) return st;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return RET_OK;
}

}  // namespace

extern "C" {

ret_status_t ret_chunkwise_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B, int N, int H,
                                       int dk, int dv, ret_dtype_t in_dt, ret_dtype_t out_dt, const float* gamma,
                                       const double* theta, int64_t pos0, int chunk, const float* state_in,
                                       float* state_out, void* stream) {
    ret_status_t st = check_common(q, k, v, o, B, N, H, dk, dv, in_dt, out_dt, gamma, theta);
    if (st != RET_OK) return st;
    if (chunk <= 0) return fail(RET_ERR_INVALID_ARG, "chunk must be positive (got %d)", chunk);
    ChunkKernels ck;
    ChunkPlan full;
    if (!resolve_chunk(in_dt, B, N, H, dk, dv, chunk, theta != nullptr, SIZE_MAX, kDefaultOpts, &ck, &full))
        return fail(RET_ERR_UNSUPPORTED, "chunkwise form: unsupported d_k=%d d_v=%d chunk=%d for %s input", dk, dv,
                    chunk, in_dt == RET_F32 ? "F32" : "BF16");
    // The library's own segment plan; its chain must fit in the scratch (the rotated copies of q and k are
    // dropped when they do not: staging then rotates, which changes only the rounding).
    if (full.chain_bytes > (size_t)RET_NOALLOC_SCRATCH_BYTES)
        return fail(RET_ERR_WORKSPACE,
                    "no-allocation chunkwise call: the segment chain of this shape needs %zu bytes, more than the "
                    "%u-byte scratch array; use ret_chunkwise_fwd with a workspace",
                    full.chain_bytes, (unsigned)RET_NOALLOC_SCRATCH_BYTES);
    const size_t avail = full.chain_bytes + full.rot_bytes <= (size_t)RET_NOALLOC_SCRATCH_BYTES
                             ? full.chain_bytes + full.rot_bytes
                             : full.chain_bytes;
    // the plan the call takes in that room: its chain must keep its counters and flags inside the region the
    // set-up zeroed
    ChunkPlan used;
    if (!resolve_chunk(in_dt, B, N, H, dk, dv, chunk, theta != nullptr, avail, kDefaultOpts, &ck, &used))
        return fail(RET_ERR_UNSUPPORTED, "chunkwise form: unsupported d_k=%d d_v=%d chunk=%d", dk, dv, chunk);
    if (used.nseg > 1 && ck.fused && !ck.split_local && !ck.fused_split &&
        chain_layout(B * H * (dv / ck.dvt), used.nseg, dk * ck.dvt).agg_off > kChainMeta)
        return fail(RET_ERR_WORKSPACE, "no-allocation chunkwise call: %d units x %d segments exceed the chain's "
                    "counter and flag region", B * H * (dv / ck.dvt), used.nseg);
    void* ws = nullptr;
    if ((st = scratch_of_device((hipStream_t)stream, &ws)) != RET_OK) return st;
    return chunkwise_run(q, k, v, o, B, N, H, dk, dv, in_dt, out_dt, gamma, theta, pos0, chunk, state_in, state_out,
                         ws, avail, stream, nullptr, nullptr, kDefaultOpts);
}

ret_timer_t* ret_timer_create(void) { return new (std::nothrow) ret_timer(); }

void ret_timer_reset(ret_timer_t* t) {
    if (!t) return;
    std::lock_guard<std::mutex> lk(t->mu);
    for (auto& r : t->recs) {
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    t->recs.clear();
}

void ret_timer_destroy(ret_timer_t* t) {
    if (!t) return;
    ret_timer_reset(t);
    delete t;
}

int ret_timer_query(ret_timer_t* t, const char* kernel, double* total_ms, int64_t* launches) {
    double tot = 0.0;
    int64_t n = 0;
    if (t) {
        std::lock_guard<std::mutex> lk(t->mu);
        for (auto& r : t->recs) {
            if (kernel && *kernel && strcmp(kernel, r.name) != 0) continue;
            if (hipEventSynchronize(r.stop) != hipSuccess) return RET_ERR_HIP;
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return RET_ERR_HIP;
            tot += ms;
            ++n;
        }
    }
    if (total_ms) *total_ms = tot;
    if (launches) *launches = n;
    return RET_OK;
}

void ret_options_default(ret_options_t* o) {
    if (!o) return;
    memset(o, 0, sizeof(*o));
    o->prerotate = -1;
    o->onchip = 1;
    o->bwd_direct = 1;
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

}  // extern "C"
