// sol_launch.h -- host-side launchers of the Sol-Attn kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sol {

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* qbar;   // [H][N][d] fp32 (unused by dense)
    const float* kbar;
    const float* vsum;
    const float* tau;    // [H][N] fp32 (unused by dense)
    const uint16_t* kbar_bf;  // [H][N][d] bf16 copy of kbar (bf16 sweep, approximate path)
    const uint16_t* vsum_bf;  // [H][N][d] bf16 copy of vsum
    void* out;
    const uint32_t* sel; // [H][N][W] selection bits of the routing kernel (bf16 sweep)
    int* queues;         // 8 per-XCD work counters (sol only)
    // bf16 sweep, query-block grouping: scratch for the partial grouping
    // costs (H * 8 * group_cost_parts(N, B) entries) and the chosen group
    // stride per head (H entries); gcost null: consecutive groups
    unsigned long long* gcost;
    int* gstride;
    int H, L, N, W;
    int nlast;           // valid tokens in the last block
    float c;             // 1/sqrt(d): proxy-score scale
    float c_log2e;       // 1/sqrt(d) * log2(e): attention logits in base 2
    int drop_approx;     // bf16 sweep: leave the unselected blocks out (keep-or-drop)
    // bf16 sweep routing inside (tau_cmp not null; sel then unused): the
    // thresholds compared with [H][N], and where the sweep writes its
    // kept counts [H][N] and, if not null, its decision bits [H][N][W]
    const float* tau_cmp;
    int32_t* kept_out;
    uint32_t* sel_out;
    // bf16 sweep, for scheduling measurements (both null in the forward pass):
    const int* order;          // [H G] group items in claim order, or null: the per-XCD queues
    unsigned long long* trace; // [H G][3] per item: claim time, end time (100 MHz clock), workgroup
};

// Each returns hipSuccess or the launch error.
hipError_t launch_pool(const void* q, const void* k, const void* v, int bf16, int H, int L,
                       int d, int B, float* qbar, float* kbar, float* vsum, uint16_t* kbar_bf,
                       uint16_t* vsum_bf, hipStream_t s);
hipError_t launch_pooled_to_bf16(const float* kbar, const float* vsum, size_t n, uint16_t* kbar_bf,
                                 uint16_t* vsum_bf, int* queues, hipStream_t s);
// Proxy rows, thresholds (computed, or taken from tau_in when it is not
// null), kept counts and selection bits (when sel is not null).
// topk >= 0: the fixed-budget comparator instead of the threshold rule
// (the k = topk largest scores of every row, ties to the lower index;
// tau = the k-th largest score); beta and tau_in are then unused.
// mom: H (d + d*d) floats of scratch for the key moments, needed when
// threshold rows are too long for LDS (N > 1280) and tau is computed.
hipError_t launch_route(const float* qbar, const float* kbar, int H, int N, int d, float c,
                        float beta, const float* tau_in, float* tau, int32_t* kept, uint32_t* sel,
                        int* queues, hipStream_t s, int topk = -1, float* mom = nullptr);
// Eq. (5) thresholds without decisions (for sweeps that route inside):
// tau [H][N] as reported, tau_cmp [H][N] the thresholds the decisions compare
// with (+inf where sigma_i = 0); mom as for launch_route; also clears the
// sweep's work counters.
hipError_t launch_thresholds(const float* qbar, const float* kbar, int H, int N, int d, float c, float beta,
                             float* tau, float* tau_cmp, float* mom, int* queues, hipStream_t s);
hipError_t launch_sweep_bf16(const AttnArgs& a, int d, int B, bool dense, hipStream_t s);
// Partial grouping costs per (head, stride) that the bf16 sweep writes.
int group_cost_parts(int N, int B);
hipError_t launch_attn_f32(const AttnArgs& a, int d, int B, bool dense, hipStream_t s);
hipError_t launch_reset_counters(int* queues, hipStream_t s);

}  // namespace sol
