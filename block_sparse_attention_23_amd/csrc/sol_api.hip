// sol_api.hip -- C ABI of libsol.so (declared in include/sol.h).
//
// Host side only: argument validation, workspace carving and kernel launches
// on the caller's stream.  No allocation, no synchronisation, no state kept
// between calls.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "sol.h"
#include "sol_launch.h"

namespace {

constexpr int kMaxBlocks = 8192;  // N bound: the proxy row lives in 32 KB of LDS
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(int H, int L, int d, int B) {
    if (H < 1 || L < 1 || d < 1 || B < 1) return SOL_EINVAL;
    if (d != 64 && d != 128) return SOL_EUNSUPPORTED;
    if (B != 32 && B != 64 && B != 128) return SOL_EUNSUPPORTED;
    const long long N = ((long long)L + B - 1) / B;
    if (N > kMaxBlocks) return SOL_EUNSUPPORTED;
    if ((long long)H * N > (1LL << 30)) return SOL_EUNSUPPORTED;
    return SOL_OK;
}

int check_tensors(const void* q, const void* k, const void* v, const void* out, sol_dtype_t dt) {
    if (dt != SOL_BF16 && dt != SOL_F32) return SOL_EINVAL;
    if (!q || !k || !v || !out) return SOL_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return SOL_EINVAL;
    return SOL_OK;
}

// Workspace layout (each region 256-byte aligned):
//   qbar, kbar, vsum : fp32 [H][N][d]     pooled tensors
//   tau              : fp32 [H][N]        thresholds
//   tau_cmp          : fp32 [H][N]        thresholds compared with, for sweeps that route inside
//   queues           : int32[8]           sweep work counters
//   gcost            : u64  [H][8][P]     partial grouping costs per head and group stride
//   gstride          : int32[H]           the group stride chosen per head
//   kbar_bf, vsum_bf : bf16 [H][N][d]     MFMA operands of the approximate path
//   sel              : u32  [H][N][W]     selection bits, W = ceil(N / 32)
//   mom              : fp32 [H][2d + d*d] key moments (routing rows longer than LDS holds)
struct Workspace {
    float* qbar;
    float* kbar;
    float* vsum;
    float* tau;
    float* tau_cmp;
    int* queues;
    unsigned long long* gcost;
    int* gstride;
    uint16_t* kbar_bf;
    uint16_t* vsum_bf;
    uint32_t* sel;
    float* mom;
    size_t bytes;
};

// lean: the layout of sol_attn_fwd_noalloc for bf16 inputs, which has no
// fp32 vsum (only the fp32 sweep reads it; the bf16 sweep reads vsum_bf).
Workspace carve(void* base, int H, int L, int d, int B, bool lean = false) {
    const size_t N = ((size_t)L + B - 1) / B;
    const size_t pooled = align_up(sizeof(float) * (size_t)H * N * d);
    const size_t pooled_bf = align_up(sizeof(uint16_t) * (size_t)H * N * d);
    const size_t taub = align_up(sizeof(float) * (size_t)H * N);
    const size_t qb = align_up(sizeof(int) * 8);
    const size_t gcb = align_up(sizeof(unsigned long long) * (size_t)H * 8 * sol::group_cost_parts((int)N, B));
    const size_t gsb = align_up(sizeof(int) * (size_t)H);
    const size_t selb = align_up(sizeof(uint32_t) * (size_t)H * N * ((N + 31) / 32));
    const size_t momb = align_up(sizeof(float) * (size_t)H * ((size_t)d + (size_t)d * d));
    char* p = static_cast<char*>(base);
    Workspace w;
    size_t off = 0;
    w.qbar = reinterpret_cast<float*>(p + off); off += pooled;
    w.kbar = reinterpret_cast<float*>(p + off); off += pooled;
    w.vsum = lean ? nullptr : reinterpret_cast<float*>(p + off); off += lean ? 0 : pooled;
    w.tau = reinterpret_cast<float*>(p + off); off += taub;
    w.tau_cmp = reinterpret_cast<float*>(p + off); off += taub;
    w.queues = reinterpret_cast<int*>(p + off); off += qb;
    w.gcost = reinterpret_cast<unsigned long long*>(p + off); off += gcb;
    w.gstride = reinterpret_cast<int*>(p + off); off += gsb;
    w.kbar_bf = reinterpret_cast<uint16_t*>(p + off); off += pooled_bf;
    w.vsum_bf = reinterpret_cast<uint16_t*>(p + off); off += pooled_bf;
    w.sel = reinterpret_cast<uint32_t*>(p + off); off += selb;
    w.mom = reinterpret_cast<float*>(p + off); off += momb;
    w.bytes = off;
    return w;
}

hipError_t launch_sweep(const sol::AttnArgs& a, int bf16, int d, int B, bool dense, hipStream_t s) {
    return bf16 ? sol::launch_sweep_bf16(a, d, B, dense, s) : sol::launch_attn_f32(a, d, B, dense, s);
}

sol::AttnArgs sweep_args(const void* q, const void* k, const void* v, const float* qbar,
                         const float* kbar, const float* vsum, const float* tau,
                         const uint16_t* kbar_bf, const uint16_t* vsum_bf, int H, int L, int d,
                         int B, void* out, int* counters, unsigned long long* gcost,
                         int* gstride, const uint32_t* sel) {
    const int N = (L + B - 1) / B;
    sol::AttnArgs a = {};
    a.q = q; a.k = k; a.v = v;
    a.qbar = qbar; a.kbar = kbar; a.vsum = vsum; a.tau = tau;
    a.kbar_bf = kbar_bf; a.vsum_bf = vsum_bf;
    a.out = out;
    a.sel = sel;
    a.queues = counters;
    a.gcost = gcost;
    a.gstride = gstride;
    a.H = H; a.L = L; a.N = N; a.W = (N + 31) / 32;
    a.nlast = L - (N - 1) * B;
    a.c = static_cast<float>(1.0 / sqrt(static_cast<double>(d)));
    a.c_log2e = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(d)));
    return a;
}

int check_forward(const void* q, const void* k, const void* v, int H, int L, int d, int B,
                  float beta, sol_dtype_t dt, const void* out, const int32_t* kept,
                  const uint32_t* sel_mask, const float* tau_out, float keep_frac, unsigned flags) {
    int st = check_shape(H, L, d, B);
    if (st != SOL_OK) return st;
    st = check_tensors(q, k, v, out, dt);
    if (st != SOL_OK) return st;
    if (!kept || !aligned(kept, 4) || isnan(beta)) return SOL_EINVAL;
    if (flags & ~(unsigned)(SOL_DROP_APPROX | SOL_TOPK | SOL_FUSED_ROUTE)) return SOL_EINVAL;
    if ((flags & SOL_TOPK) && (flags & SOL_FUSED_ROUTE)) return SOL_EINVAL;
    if ((flags & SOL_TOPK) && !(keep_frac >= 0.0f && keep_frac <= 1.0f)) return SOL_EINVAL;
    if (flags && dt != SOL_BF16) return SOL_EUNSUPPORTED;
    if ((sel_mask && !aligned(sel_mask, 4)) || (tau_out && !aligned(tau_out, 4))) return SOL_EINVAL;
    return SOL_OK;
}

// pool -> route -> sweep on the stream, with the workspace regions of w
int launch_forward(const void* q, const void* k, const void* v, int H, int L, int d, int B,
                   float beta, sol_dtype_t dt, void* out, int32_t* kept, const Workspace& w,
                   void* stream, uint32_t* sel_mask, float* tau_out, float keep_frac, unsigned flags) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int N = (L + B - 1) / B;
    const int bf16 = dt == SOL_BF16;
    const float c = static_cast<float>(1.0 / sqrt(static_cast<double>(d)));
    // The thresholds and selection bits go straight to the caller's arrays
    // when it asks for them.
    float* tau = tau_out ? tau_out : w.tau;
    uint32_t* sel = sel_mask ? sel_mask : w.sel;

    if (sol::launch_pool(q, k, v, bf16, H, L, d, B, w.qbar, w.kbar, w.vsum,
                         bf16 ? w.kbar_bf : nullptr, bf16 ? w.vsum_bf : nullptr, s) != hipSuccess)
        return SOL_EHIP;
    if (flags & SOL_FUSED_ROUTE) {
        // thresholds first; the sweep routes, counts and (if asked) records
        // its decisions itself
        if (sol::launch_thresholds(w.qbar, w.kbar, H, N, d, c, beta, tau, w.tau_cmp, w.mom, w.queues, s) !=
            hipSuccess)
            return SOL_EHIP;
        sol::AttnArgs a = sweep_args(q, k, v, w.qbar, w.kbar, w.vsum, tau, w.kbar_bf, w.vsum_bf, H, L,
                                     d, B, out, w.queues, nullptr, nullptr, nullptr);
        a.tau_cmp = w.tau_cmp;
        a.kept_out = kept;
        a.sel_out = sel_mask;
        a.drop_approx = (flags & SOL_DROP_APPROX) ? 1 : 0;
        if (launch_sweep(a, bf16, d, B, false, s) != hipSuccess) return SOL_EHIP;
        return SOL_OK;
    }
    // fixed budget: round(keep_frac * N), halves up, within [0, N]
    const int topk = (flags & SOL_TOPK)
                         ? static_cast<int>(fmin((double)N, fmax(0.0, floor((double)keep_frac * N + 0.5))))
                         : -1;
    // (the routing kernel also clears the sweep's work counters)
    if (sol::launch_route(w.qbar, w.kbar, H, N, d, c, beta, nullptr, tau, kept, sel, w.queues, s,
                          topk, w.mom) != hipSuccess)
        return SOL_EHIP;
    sol::AttnArgs a = sweep_args(q, k, v, w.qbar, w.kbar, w.vsum, tau, w.kbar_bf, w.vsum_bf, H, L,
                                 d, B, out, w.queues, w.gcost, w.gstride, sel);
    a.drop_approx = (flags & SOL_DROP_APPROX) ? 1 : 0;
    if (launch_sweep(a, bf16, d, B, false, s) != hipSuccess) return SOL_EHIP;
    return SOL_OK;
}

int forward(const void* q, const void* k, const void* v, int H, int L, int d, int B, float beta,
            sol_dtype_t dt, void* out, int32_t* kept, void* ws, size_t ws_bytes, void* stream,
            uint32_t* sel_mask, float* tau_out, float keep_frac = 0.0f, unsigned flags = 0u) {
    const int st = check_forward(q, k, v, H, L, d, B, beta, dt, out, kept, sel_mask, tau_out,
                                 keep_frac, flags);
    if (st != SOL_OK) return st;
    if (!ws || !aligned(ws, kAlign)) return SOL_EWORKSPACE;
    const Workspace w = carve(ws, H, L, d, B);
    if (ws_bytes < w.bytes) return SOL_EWORKSPACE;
    return launch_forward(q, k, v, H, L, d, B, beta, dt, out, kept, w, stream, sel_mask, tau_out,
                          keep_frac, flags);
}

// ---------------------------------------------------------------------------
// The allocation-free forward pass (sol_attn_fwd_noalloc): its workspace is
// this static device array, one copy per GPU, which each GPU holds from the
// library's first use on it until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: the kernels receive the
// device address that hipGetSymbolAddress returns for the current device,
// looked up once per device and kept in scratch_addr.  Every call on a GPU
// shares that GPU's copy; the kernels write every region before reading it
// (the routing kernel clears the work counters), so nothing is left over
// from an earlier call.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SOL_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_addr[kMaxDevices];  // device address of `scratch` per device, once looked up

// The device address of `scratch` on the device of `stream` (the current
// device for the null stream): looked up with that device current on the
// first call for the device, then reused.
int scratch_on(hipStream_t stream, void** addr) {
    int dev = -1;
    if (stream) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return SOL_EHIP;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return SOL_EHIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return SOL_EHIP;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_addr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return SOL_EHIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return SOL_EHIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return SOL_EHIP;
        if (e != hipSuccess || !p) return SOL_EHIP;
        scratch_addr[dev] = p;
    }
    *addr = scratch_addr[dev];
    return SOL_OK;
}

}  // namespace

extern "C" {

size_t sol_workspace_bytes(int H, int L, int d, int B) {
    if (check_shape(H, L, d, B) != SOL_OK) return 0;
    return carve(nullptr, H, L, d, B).bytes;
}

int sol_pool(const void* q, const void* k, const void* v, int H, int L, int d, int B, sol_dtype_t dt,
             float* qbar, float* kbar, float* vsum, void* stream) {
    int st = check_shape(H, L, d, B);
    if (st != SOL_OK) return st;
    if (dt != SOL_BF16 && dt != SOL_F32) return SOL_EINVAL;
    if (!q || !k || !v || !qbar || !kbar || !vsum) return SOL_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(qbar, 4) ||
        !aligned(kbar, 4) || !aligned(vsum, 4))
        return SOL_EINVAL;
    if (sol::launch_pool(q, k, v, dt == SOL_BF16, H, L, d, B, qbar, kbar, vsum, nullptr, nullptr,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
        return SOL_EHIP;
    return SOL_OK;
}

int sol_route(const float* qbar, const float* kbar, int H, int L, int d, int B, float beta,
              float* tau, int32_t* kept_counts, uint32_t* sel_bits, void* workspace,
              size_t ws_bytes, void* stream) {
    int st = check_shape(H, L, d, B);
    if (st != SOL_OK) return st;
    if (!qbar || !kbar || !tau || !kept_counts || isnan(beta)) return SOL_EINVAL;
    if (!aligned(qbar, 16) || !aligned(kbar, 16) || !aligned(tau, 4) || !aligned(kept_counts, 4) ||
        (sel_bits && !aligned(sel_bits, 4)))
        return SOL_EINVAL;
    if (!workspace || !aligned(workspace, kAlign)) return SOL_EWORKSPACE;
    const Workspace w = carve(workspace, H, L, d, B);
    if (ws_bytes < w.bytes) return SOL_EWORKSPACE;
    const int N = (L + B - 1) / B;
    const float c = static_cast<float>(1.0 / sqrt(static_cast<double>(d)));
    if (sol::launch_route(qbar, kbar, H, N, d, c, beta, nullptr, tau, kept_counts, sel_bits, nullptr,
                          static_cast<hipStream_t>(stream), -1, w.mom) != hipSuccess)
        return SOL_EHIP;
    return SOL_OK;
}

int sol_sweep(const void* q, const void* k, const void* v, const float* qbar, const float* kbar,
              const float* vsum, const float* tau, int H, int L, int d, int B, sol_dtype_t dt,
              void* out, void* workspace, size_t ws_bytes, const uint32_t* sel_bits,
              uint32_t* sel_mask, void* stream) {
    int st = check_shape(H, L, d, B);
    if (st != SOL_OK) return st;
    st = check_tensors(q, k, v, out, dt);
    if (st != SOL_OK) return st;
    if (!qbar || !kbar || !vsum || !tau) return SOL_EINVAL;
    if (!aligned(qbar, 16) || !aligned(kbar, 16) || !aligned(vsum, 16) || !aligned(tau, 4) ||
        (sel_mask && !aligned(sel_mask, 4)) || (sel_bits && !aligned(sel_bits, 4)))
        return SOL_EINVAL;
    if (!workspace || !aligned(workspace, kAlign)) return SOL_EWORKSPACE;
    const Workspace w = carve(workspace, H, L, d, B);
    if (ws_bytes < w.bytes) return SOL_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int N = (L + B - 1) / B;
    const int bf16 = dt == SOL_BF16;
    // bf16 operands of the approximate path (and cleared work counters)
    if (bf16) {
        if (sol::launch_pooled_to_bf16(kbar, vsum, (size_t)H * N * d, w.kbar_bf, w.vsum_bf,
                                       w.queues, s) != hipSuccess)
            return SOL_EHIP;
    } else if (sol::launch_reset_counters(w.queues, s) != hipSuccess) {
        return SOL_EHIP;
    }
    // selection bits against the caller's thresholds: the caller's, or
    // derived here (and copied to sel_mask when it asks for them)
    const size_t nsel = (size_t)H * N * ((N + 31) / 32);
    const uint32_t* sel = sel_bits;
    if (sel_bits && sel_mask &&
        hipMemcpyAsync(sel_mask, sel_bits, nsel * sizeof(uint32_t), hipMemcpyDeviceToDevice, s) !=
            hipSuccess)
        return SOL_EHIP;
    if (!sel) {
        uint32_t* dst = sel_mask ? sel_mask : w.sel;
        const float c = static_cast<float>(1.0 / sqrt(static_cast<double>(d)));
        if (sol::launch_route(qbar, kbar, H, N, d, c, 0.0f, tau, nullptr, nullptr, dst, nullptr, s) !=
            hipSuccess)
            return SOL_EHIP;
        sel = dst;
    }
    const sol::AttnArgs a = sweep_args(q, k, v, qbar, kbar, vsum, tau, w.kbar_bf, w.vsum_bf, H, L,
                                       d, B, out, w.queues, w.gcost, w.gstride, sel);
    if (launch_sweep(a, bf16, d, B, false, s) != hipSuccess) return SOL_EHIP;
    return SOL_OK;
}

int sol_sweep_timed(const void* q, const void* k, const void* v, const float* qbar, const float* kbar,
                    const float* vsum, const float* tau, int H, int L, int d, int B, sol_dtype_t dt,
                    void* out, void* workspace, size_t ws_bytes, const uint32_t* sel_bits,
                    const int32_t* order, uint64_t* item_clock, void* stream) {
    int st = check_shape(H, L, d, B);
    if (st != SOL_OK) return st;
    st = check_tensors(q, k, v, out, dt);
    if (st != SOL_OK) return st;
    if (dt != SOL_BF16) return SOL_EUNSUPPORTED;
    if (!qbar || !kbar || !vsum || !tau || !sel_bits || !item_clock) return SOL_EINVAL;
    if (!aligned(qbar, 16) || !aligned(kbar, 16) || !aligned(vsum, 16) || !aligned(tau, 4) ||
        !aligned(sel_bits, 4) || (order && !aligned(order, 4)) || !aligned(item_clock, 8))
        return SOL_EINVAL;
    if (!workspace || !aligned(workspace, kAlign)) return SOL_EWORKSPACE;
    const Workspace w = carve(workspace, H, L, d, B);
    if (ws_bytes < w.bytes) return SOL_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int N = (L + B - 1) / B;
    // bf16 operands of the approximate path; the kernel clears the work counters
    if (sol::launch_pooled_to_bf16(kbar, vsum, (size_t)H * N * d, w.kbar_bf, w.vsum_bf, w.queues, s) !=
        hipSuccess)
        return SOL_EHIP;
    sol::AttnArgs a = sweep_args(q, k, v, qbar, kbar, vsum, tau, w.kbar_bf, w.vsum_bf, H, L, d, B, out,
                                 w.queues, w.gcost, w.gstride, sel_bits);
    a.order = order;
    a.trace = reinterpret_cast<unsigned long long*>(item_clock);
    if (launch_sweep(a, 1, d, B, false, s) != hipSuccess) return SOL_EHIP;
    return SOL_OK;
}

int sol_attn_fwd(const void* q, const void* k, const void* v, int H, int L, int d, int B, float beta,
                 sol_dtype_t dt, void* out, int32_t* kept_counts, void* workspace, size_t ws_bytes,
                 void* stream) {
    return forward(q, k, v, H, L, d, B, beta, dt, out, kept_counts, workspace, ws_bytes, stream,
                   nullptr, nullptr);
}

int sol_attn_fwd_dbg(const void* q, const void* k, const void* v, int H, int L, int d, int B,
                     float beta, sol_dtype_t dt, void* out, int32_t* kept_counts, void* workspace,
                     size_t ws_bytes, void* stream, uint32_t* sel_mask, float* tau) {
    return forward(q, k, v, H, L, d, B, beta, dt, out, kept_counts, workspace, ws_bytes, stream,
                   sel_mask, tau);
}

int sol_attn_fwd_variant(const void* q, const void* k, const void* v, int H, int L, int d, int B,
                         float beta, float keep_frac, unsigned flags, sol_dtype_t dt, void* out,
                         int32_t* kept_counts, void* workspace, size_t ws_bytes, void* stream,
                         uint32_t* sel_mask, float* tau) {
    return forward(q, k, v, H, L, d, B, beta, dt, out, kept_counts, workspace, ws_bytes, stream,
                   sel_mask, tau, keep_frac, flags);
}

int sol_attn_dense(const void* q, const void* k, const void* v, int H, int L, int d, sol_dtype_t dt,
                   void* out, void* stream) {
    const int B = 64;
    int st = check_shape(H, L, d, B);
    if (st != SOL_OK) return st;
    st = check_tensors(q, k, v, out, dt);
    if (st != SOL_OK) return st;
    const int N = (L + B - 1) / B;
    sol::AttnArgs a = {};
    a.q = q; a.k = k; a.v = v;
    a.out = out;
    a.H = H; a.L = L; a.N = N; a.W = (N + 31) / 32;
    a.nlast = L - (N - 1) * B;
    a.c = static_cast<float>(1.0 / sqrt(static_cast<double>(d)));
    a.c_log2e = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(d)));
    if (launch_sweep(a, dt == SOL_BF16, d, B, true, static_cast<hipStream_t>(stream)) != hipSuccess)
        return SOL_EHIP;
    return SOL_OK;
}

int sol_attn_fwd_noalloc(const void* q, const void* k, const void* v, int H, int L, int d, int B,
                         float beta, sol_dtype_t dt, void* out, int32_t* kept_counts, void* stream) {
    int st = check_forward(q, k, v, H, L, d, B, beta, dt, out, kept_counts, nullptr, nullptr, 0.0f, 0u);
    if (st != SOL_OK) return st;
    const bool lean = dt == SOL_BF16;
    if (carve(nullptr, H, L, d, B, lean).bytes > SOL_NOALLOC_SCRATCH_BYTES) return SOL_ESCRATCH;
    void* base = nullptr;
    st = scratch_on(static_cast<hipStream_t>(stream), &base);
    if (st != SOL_OK) return st;
    return launch_forward(q, k, v, H, L, d, B, beta, dt, out, kept_counts, carve(base, H, L, d, B, lean),
                          stream, nullptr, nullptr, 0.0f, 0u);
}

const char* sol_status_string(int status) {
    switch (status) {
        case SOL_OK: return "success";
        case SOL_EINVAL: return "invalid argument (null or misaligned pointer, bad size, NaN beta or bad dtype)";
        case SOL_EUNSUPPORTED: return "unsupported shape (d must be 64 or 128, B 32, 64 or 128; N <= 8192)";
        case SOL_EWORKSPACE: return "workspace missing, misaligned or smaller than sol_workspace_bytes()";
        case SOL_EHIP: return "HIP kernel launch failed";
        case SOL_ESCRATCH:
            return "problem too large for the static scratch of sol_attn_fwd_noalloc "
                   "(SOL_NOALLOC_SCRATCH_BYTES); use sol_attn_fwd with a workspace";
        default: return "unknown status";
    }
}

}  // extern "C"
