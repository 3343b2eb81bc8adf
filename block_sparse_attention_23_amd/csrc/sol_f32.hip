// sol_f32.hip -- the Sol-Attn sweep for fp32 inputs (vector ALU, fp32
// arithmetic throughout; the path that meets the fp32 tolerance).  Like the
// bf16 sweep it takes its decisions from the routing kernel's bits; the
// merge is the bf16 sweep's.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sol_device.h"
#include "sol_launch.h"

namespace sol {

// ============================================================================
// attention sweep, fp32 inputs (vector ALU; exact fp32 arithmetic path)
// ============================================================================
// Four consecutive lanes own one query row; lane quarter qq holds d/4 of its
// query and output columns.
template <int D, int BLK, bool DENSE>
__global__ void __launch_bounds__(4 * BLK) attn_f32_kernel(AttnArgs a) {
    constexpr int NT = 4 * BLK;
    constexpr int Q4 = D / 4;
    constexpr int KP = D + 4;  // pitch keeps 16-byte alignment
    __shared__ __align__(16) float Kf[BLK * KP];
    __shared__ __align__(16) float Vf[BLK * KP];
    __shared__ float wt_s[BLK];            // column weight; 0 = masked column
    __shared__ int sel_list[BLK];
    __shared__ unsigned char flag_s[BLK];
    __shared__ int misc_s[2];

    const float* __restrict__ qg = static_cast<const float*>(a.q);
    const float* __restrict__ kg = static_cast<const float*>(a.k);
    const float* __restrict__ vg = static_cast<const float*>(a.v);
    float* __restrict__ og = static_cast<float*>(a.out);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rr = tid >> 2, qq = tid & 3;
    const int H = a.H, L = a.L, N = a.N;

    int dense_item = -1;
    if (DENSE) {
        const int total = H * N;
        const int per = (total + 7) / 8;
        const int idx = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
        if ((int)(blockIdx.x >> 3) >= per || idx >= total) return;
        dense_item = idx;
    }

    for (;;) {
        int item;
        if (DENSE) {
            item = dense_item;
        } else {
            __syncthreads();
            if (tid == 0) misc_s[0] = claim_item(a.queues, H, N);
            __syncthreads();
            item = misc_s[0];
            if (item < 0) break;
        }
        const int h = item / N, i = item % N;
        const size_t head_off = (size_t)h * L * D;
        const int row = i * BLK + rr;

        float qr[Q4];
        {
            const float4* src = reinterpret_cast<const float4*>(qg + head_off + (size_t)min(row, L - 1) * D + qq * Q4);
#pragma unroll
            for (int e = 0; e < Q4 / 4; ++e) {
                const float4 t = src[e];
                qr[4 * e] = t.x; qr[4 * e + 1] = t.y; qr[4 * e + 2] = t.z; qr[4 * e + 3] = t.w;
            }
        }
        const uint32_t* srow = DENSE ? nullptr : a.sel + (size_t)item * a.W;  // bit j: s_ij > tau_i
        float m_run = -INFINITY, l_run = 0.0f;
        float acc[Q4];
#pragma unroll
        for (int e = 0; e < Q4; ++e) acc[e] = 0.0f;

        // one tile of BLK columns already staged in Kf / Vf / wt_s
        auto tile = [&]() {
            float x[BLK];
            float mx = -INFINITY;
#pragma unroll 8
            for (int t = 0; t < BLK; ++t) {
                const float* kr = Kf + t * KP + qq * Q4;
                float p = 0.0f;
#pragma unroll
                for (int e = 0; e < Q4; ++e) p = __builtin_fmaf(qr[e], kr[e], p);
                const float p01 = p + quad_xor1(p);
                const float s = p01 + quad_xor2(p01);
                x[t] = wt_s[t] > 0.0f ? s * a.c_log2e : -INFINITY;
                mx = fmaxf(mx, x[t]);
            }
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
            const float alpha = exp2f(m_run - m_use);
            l_run *= alpha;
#pragma unroll
            for (int e = 0; e < Q4; ++e) acc[e] *= alpha;
#pragma unroll 8
            for (int t = 0; t < BLK; ++t) {
                const float p = exp2f(x[t] - m_use);
                l_run = __builtin_fmaf(wt_s[t], p, l_run);
                const float* vr = Vf + t * KP + qq * Q4;
#pragma unroll
                for (int e = 0; e < Q4; ++e) acc[e] = __builtin_fmaf(p, vr[e], acc[e]);
            }
            m_run = m_new;
        };

        const int nch = (N + BLK - 1) / BLK;
        for (int ch = 0; ch < nch; ++ch) {
            const int j0 = ch * BLK;
            const int nj = min(BLK, N - j0);
            int nex = nj;
            if (!DENSE) {
                __syncthreads();
                {
                    const int jj = rr;
                    const int jc = min(j0 + jj, N - 1);
                    const bool valid = jj < nj;
                    float kv[D / 4];
                    load_kbar_quarter<D>(a.kbar + ((size_t)h * N + jc) * D, qq, kv);
                    const int jg = j0 + jj;
                    const bool sel = valid && ((srow[jg >> 5] >> (jg & 31)) & 1u);
                    if (qq == 0) {
                        flag_s[jj] = sel ? 1 : (valid ? 0 : 2);
                        wt_s[jj] = (valid && !sel)
                                       ? static_cast<float>((j0 + jj == N - 1) ? a.nlast : BLK)
                                       : 0.0f;
                    }
                    float vv[D / 4];
                    load_kbar_quarter<D>(a.vsum + ((size_t)h * N + jc) * D, qq, vv);
#pragma unroll
                    for (int e = 0; e < Q4; ++e) {
                        Kf[jj * KP + qq * Q4 + e] = valid ? kv[e] : 0.0f;
                        Vf[jj * KP + qq * Q4 + e] = valid ? vv[e] : 0.0f;
                    }
                }
                __syncthreads();
                if (wave == 0) {
                    int base = 0;
                    for (int hh = 0; hh < (BLK + 63) / 64; ++hh) {
                        const int jj = hh * 64 + lane;
                        const bool sel = jj < BLK && flag_s[jj] == 1;
                        const uint64_t msk = __ballot(sel);
                        const int pos = base + __popcll(msk & ((1ull << lane) - 1ull));
                        if (sel) sel_list[pos] = j0 + jj;
                        base += __popcll(msk);
                    }
                    if (lane == 0) misc_s[1] = base;
                }
                __syncthreads();
                nex = misc_s[1];
                if (nex < nj) tile();
            }
            for (int e = 0; e < nex; ++e) {
                const int j = DENSE ? j0 + e : sel_list[e];
                __syncthreads();
                const int t0 = j * BLK;
                for (int c = tid; c < BLK * (D / 4); c += NT) {
                    const int r = c / (D / 4), col = (c % (D / 4)) * 4;
                    float4 kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
                    if (t0 + r < L) {
                        kk = *reinterpret_cast<const float4*>(kg + head_off + (size_t)(t0 + r) * D + col);
                        vv = *reinterpret_cast<const float4*>(vg + head_off + (size_t)(t0 + r) * D + col);
                    }
                    *reinterpret_cast<float4*>(Kf + r * KP + col) = kk;
                    *reinterpret_cast<float4*>(Vf + r * KP + col) = vv;
                }
                for (int t = tid; t < BLK; t += NT) wt_s[t] = (t0 + t < L) ? 1.0f : 0.0f;
                __syncthreads();
                tile();
            }
        }
        const float inv = 1.0f / l_run;
        if (row < L) {
            float4* dst = reinterpret_cast<float4*>(og + head_off + (size_t)row * D + qq * Q4);
#pragma unroll
            for (int e = 0; e < Q4 / 4; ++e)
                dst[e] = float4{acc[4 * e] * inv, acc[4 * e + 1] * inv, acc[4 * e + 2] * inv,
                                acc[4 * e + 3] * inv};
        }
        if (DENSE) break;
    }
}

namespace {

int cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}

template <int D, int BLK, bool DENSE>
hipError_t f32_t(const AttnArgs& a, hipStream_t s) {
    auto kern = attn_f32_kernel<D, BLK, DENSE>;
    const int threads = 4 * BLK;
    int grid;
    if (DENSE) {
        grid = 8 * ((a.H * a.N + 7) / 8);
    } else {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        grid = cu_count() * per_cu;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, int d, int B, bool dense, hipStream_t s) {
    if (d == 64 && B == 32 && !dense) return f32_t<64, 32, false>(a, s);
    if (d == 128 && B == 32 && !dense) return f32_t<128, 32, false>(a, s);
    if (d == 64 && B == 64) return dense ? f32_t<64, 64, true>(a, s) : f32_t<64, 64, false>(a, s);
    if (d == 64 && B == 128) return dense ? f32_t<64, 128, true>(a, s) : f32_t<64, 128, false>(a, s);
    if (d == 128 && B == 64) return dense ? f32_t<128, 64, true>(a, s) : f32_t<128, 64, false>(a, s);
    if (d == 128 && B == 128) return dense ? f32_t<128, 128, true>(a, s) : f32_t<128, 128, false>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace sol
