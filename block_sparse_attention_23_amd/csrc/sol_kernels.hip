// sol_kernels.hip -- Sol-Attn kernels for MI355X (gfx950, CDNA4).
//
// Stages of one forward pass ("Sol-Attn" visual explainer, "The complete
// idea in one pass"):
//   pool   -- one pass over Q, K, V: block means of Q and K, block sums of V.
//   route  -- per (head, query block): the proxy-score row over all N key
//             blocks, held in LDS only; its population mean and standard
//             deviation give tau = mu + beta*sigma (Eq. (4), Eq. (5)).
//   attn   -- the fused sweep.  For each query block it streams the pooled
//             keys chunk by chunk, recomputes each chunk's proxy scores with
//             the routing kernel's own arithmetic, compares them with tau,
//             folds the unselected columns of the chunk in through the
//             token-to-pooled-key tile Q_i Kbar^T (Eq. (9), Eq. (10),
//             Eq. (11)), and computes the selected key blocks exactly; both
//             paths update one running max / denominator / accumulator.
//
// Layouts: token tensors [H][L][d]; pooled tensors [H][N][d] fp32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sol_device.h"
#include "sol_launch.h"

namespace sol {

// ============================================================================
// pool
// ============================================================================
// One workgroup per (head, block).  Thread t reads 16-byte vectors of a row
// (VEC elements) at column chunk t % CH, rows t / CH, t / CH + RG, ...; the RG
// row-group partial sums are then added in a fixed order through LDS.
template <typename T, int D, int BLK>
__global__ void __launch_bounds__(256) pool_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, int L, int N,
                                                   float* __restrict__ qbar,
                                                   float* __restrict__ kbar,
                                                   float* __restrict__ vsum) {
    constexpr int VEC = 16 / sizeof(T);
    constexpr int CH = D / VEC;
    constexpr int RG = 256 / CH;
    constexpr int IT = (BLK + RG - 1) / RG;
    __shared__ float red[3][RG][D + 1];

    const int item = blockIdx.x;  // h * N + j
    const int h = item / N, j = item % N;
    const int t0 = j * BLK;
    const int n = min(BLK, L - t0);
    const int tid = threadIdx.x;
    const int ch = tid % CH, rg = tid / CH;

    float aq[VEC], ak[VEC], av[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) aq[e] = ak[e] = av[e] = 0.0f;

    const size_t base = ((size_t)h * L + t0) * D + ch * VEC;
    u32x4_t bq[IT], bk[IT], bv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int r = rg + it * RG;
        if (r < n) {
            bq[it] = *reinterpret_cast<const u32x4_t*>(q + base + (size_t)r * D);
            bk[it] = *reinterpret_cast<const u32x4_t*>(k + base + (size_t)r * D);
            bv[it] = *reinterpret_cast<const u32x4_t*>(v + base + (size_t)r * D);
        } else {
            bq[it] = bk[it] = bv[it] = u32x4_t{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float xq, xk, xv;
            if constexpr (sizeof(T) == 2) {
                const uint32_t wq = bq[it][e / 2], wk = bk[it][e / 2], wv = bv[it][e / 2];
                const int sh = (e & 1) ? 16 : 0;
                xq = bf16_bits_to_f32(static_cast<u16>(wq >> sh));
                xk = bf16_bits_to_f32(static_cast<u16>(wk >> sh));
                xv = bf16_bits_to_f32(static_cast<u16>(wv >> sh));
            } else {
                xq = __uint_as_float(bq[it][e]);
                xk = __uint_as_float(bk[it][e]);
                xv = __uint_as_float(bv[it][e]);
            }
            aq[e] += xq;
            ak[e] += xk;
            av[e] += xv;
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        red[0][rg][ch * VEC + e] = aq[e];
        red[1][rg][ch * VEC + e] = ak[e];
        red[2][rg][ch * VEC + e] = av[e];
    }
    __syncthreads();
    const float inv_n = 1.0f / static_cast<float>(n);
    for (int x = tid; x < 3 * D; x += 256) {
        const int which = x / D, col = x % D;
        float s = 0.0f;
#pragma unroll
        for (int r = 0; r < RG; ++r) s += red[which][r][col];
        const size_t o = (size_t)item * D + col;
        if (which == 0) qbar[o] = s * inv_n;
        else if (which == 1) kbar[o] = s * inv_n;
        else vsum[o] = s;
    }
}

// ============================================================================
// route
// ============================================================================
// Deterministic sum over a 256-thread workgroup: butterfly inside each wave
// (every lane ends with the same value), then the four wave sums in a fixed
// order.
__device__ __forceinline__ float block_sum256(float x, float* red4) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = x;
    __syncthreads();
    return (red4[0] + red4[1]) + (red4[2] + red4[3]);
}

// One workgroup (256 threads) per (head h, query block i).  The proxy row
// s_i. (N floats) lives in dynamic LDS only.  Writes tau_i and the kept
// count |{j : s_ij > tau_i}|.  When `queues` is given, workgroup 0 also
// resets the sweep's eight work counters (the forward pass launches the
// sweep right after this kernel on the same stream).
template <int D>
__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ qbar,
                                                    const float* __restrict__ kbar, int N,
                                                    float c, float beta,
                                                    float* __restrict__ tau_out,
                                                    int32_t* __restrict__ kept,
                                                    int* __restrict__ queues) {
    extern __shared__ float row[];
    __shared__ float qb[D];
    __shared__ float red4[4];
    const int item = blockIdx.x;
    const int h = item / N;
    const int tid = threadIdx.x;
    if (queues && item == 0 && tid < 8) queues[tid] = 0;
    for (int t = tid; t < D; t += 256) qb[t] = qbar[(size_t)item * D + t];
    __syncthreads();

    const int jj = tid >> 2, qq = tid & 3;
    for (int j0 = 0; j0 < N; j0 += 64) {
        const int j = j0 + jj;
        float kv[D / 4];
        load_kbar_quarter<D>(kbar + ((size_t)h * N + min(j, N - 1)) * D, qq, kv);
        const float s = proxy_from_quarter<D>(qb, kv, qq, c);
        if (qq == 0 && j < N) row[j] = s;
    }
    __syncthreads();

    float part = 0.0f;
    for (int j = tid; j < N; j += 256) part += row[j];
    const float mu = block_sum256(part, red4) / static_cast<float>(N);
    part = 0.0f;
    for (int j = tid; j < N; j += 256) {
        const float dlt = row[j] - mu;
        part = __builtin_fmaf(dlt, dlt, part);
    }
    const float var = block_sum256(part, red4) / static_cast<float>(N);
    const float sigma = sqrtf(fmaxf(var, 0.0f));
    float tau;
    if (isinf(beta)) tau = beta;  // -inf: every block exact; +inf: none
    else tau = __builtin_fmaf(beta, sigma, mu);
    float cnt = 0.0f;
    for (int j = tid; j < N; j += 256) cnt += (row[j] > tau) ? 1.0f : 0.0f;
    const float total = block_sum256(cnt, red4);
    if (tid == 0) {
        tau_out[item] = tau;
        kept[item] = static_cast<int32_t>(total);
    }
}

__global__ void reset_counters_kernel(int* queues) {
    if (threadIdx.x < 8) queues[threadIdx.x] = 0;
}

// ============================================================================
// attention sweep, bf16 inputs, MFMA (v_mfma_f32_16x16x32_bf16)
// ============================================================================
// One workgroup owns one query block of BLK rows at a time; wave w owns rows
// 16w .. 16w+15.  Scores are formed transposed, S^T = K Q^T, so that each
// lane holds one query row (l % 16) and 4 keys per 16-key tile; the softmax
// weights then feed the P V product (O^T = V^T P^T) straight from registers.
// K tiles sit in LDS row-major ([key][d], padded pitch); V tiles are stored
// transposed ([d][key]) while they are staged.  fp32 accumulation; the
// probabilities are rounded to bf16 for the P V product.
//
// Scheduling (sol): persistent workgroups; eight work queues, one per XCD
// (workgroup w runs on XCD w % 8).  Queue x holds, head by head, the query
// blocks [x N / 8, (x+1) N / 8) so that the workgroups of one XCD work on
// neighbouring query blocks of the same head at the same time (their exact
// key blocks overlap and hit that XCD's L2).  A workgroup whose queue is empty
// takes work from the next queue; every workgroup exits once all eight
// queues are drained.  Dense: one workgroup per query block, XCD-contiguous.
__device__ __forceinline__ int claim_item(int* queues, int H, int N) {
    const int xcd = blockIdx.x & 7;
#pragma unroll 1
    for (int t = 0; t < 8; ++t) {
        const int x = (xcd + t) & 7;
        const int lo = (x * N) >> 3, hi = ((x + 1) * N) >> 3;
        const int nx = hi - lo;
        if (nx == 0) continue;
        const int kk = atomicAdd(&queues[x], 1);
        if (kk < H * nx) return (kk / nx) * N + lo + (kk % nx);
    }
    return -1;
}

template <int D, int BLK>
struct Bf16Tile {
    static constexpr int NT = 4 * BLK;   // threads
    static constexpr int KP = D + 8;     // K pitch (bf16 elements)
    static constexpr int VP = BLK + 8;   // V^T pitch
    static constexpr int NKT = BLK / 16; // 16-key tiles
    static constexpr int NDT = D / 16;   // 16-wide d tiles of the output
    static constexpr int NS = D / 32;    // 32-deep k-steps over d
};

// S^T tile (BLK keys x 16 queries of this wave) from Ks and the Q fragments.
template <int D, int BLK>
__device__ __forceinline__ void scores_t(const u16* Ks, const bf16x8_t (&qf)[D / 32],
                                         f32x4_t (&sacc)[BLK / 16], int l16, int g) {
    using T = Bf16Tile<D, BLK>;
#pragma unroll
    for (int kt = 0; kt < T::NKT; ++kt) sacc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < T::NS; ++s) {
#pragma unroll
        for (int kt = 0; kt < T::NKT; ++kt) {
            const u32x4_t av =
                *reinterpret_cast<const u32x4_t*>(Ks + (kt * 16 + l16) * T::KP + s * 32 + g * 8);
            sacc[kt] = mfma16(as_bf16x8(av), qf[s], sacc[kt]);
        }
    }
}

// Online-softmax update with the logits x (base-2 units, -inf = masked) and
// per-key weights w (n_j for pooled keys, 1 for tokens), then O += V^T P^T.
template <int D, int BLK>
__device__ __forceinline__ void softmax_pv(float (&x)[BLK / 16][4], const float (&w)[BLK / 16][4],
                                           const u16* Vt, float& m_run, float& l_run,
                                           f32x4_t (&o)[D / 16], int l16, int g) {
    using T = Bf16Tile<D, BLK>;
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < T::NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, x[kt][r]);
    mx = wave_max_xor16_32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < T::NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            x[kt][r] = __builtin_amdgcn_exp2f(x[kt][r] - m_use);
            psum = __builtin_fmaf(w[kt][r], x[kt][r], psum);
        }
    l_run = __builtin_fmaf(l_run, alpha, psum);
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < T::NDT; ++dt) o[dt] *= alpha;
    // P^T operand: k-index 8g+e of k-step u is key 32u + 4g + e (e < 4) or
    // 32u + 16 + 4g + (e - 4) (e >= 4) -- the keys this lane already holds.
#pragma unroll
    for (int u = 0; u < BLK / 32; ++u) {
        const u32x4_t pb = {pack_bf16x2(x[2 * u][0], x[2 * u][1]),
                            pack_bf16x2(x[2 * u][2], x[2 * u][3]),
                            pack_bf16x2(x[2 * u + 1][0], x[2 * u + 1][1]),
                            pack_bf16x2(x[2 * u + 1][2], x[2 * u + 1][3])};
#pragma unroll
        for (int dt = 0; dt < T::NDT; ++dt) {
            const u16* vr = Vt + (dt * 16 + l16) * T::VP + 32 * u + 4 * g;
            const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vr);
            const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vr + 16);
            const u32x4_t av = {lo[0], lo[1], hi[0], hi[1]};
            o[dt] = mfma16(as_bf16x8(av), as_bf16x8(pb), o[dt]);
        }
    }
}

// Stage key block j (K row-major, V transposed) into LDS; rows past L are 0.
template <int D, int BLK>
__device__ __forceinline__ void stage_kv(const u16* __restrict__ k, const u16* __restrict__ v,
                                         size_t head_off, int L, int j, u16* Ks, u16* Vt,
                                         int tid) {
    using T = Bf16Tile<D, BLK>;
    constexpr int KCH = BLK * D / 8;                  // 16-byte chunks of K
    constexpr int KIT = (KCH + T::NT - 1) / T::NT;
    const int t0 = j * BLK;
    u32x4_t kr[KIT];
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
        const int c = tid + it * T::NT;
        const int r = c / (D / 8), col = (c % (D / 8)) * 8;
        kr[it] = (c < KCH && t0 + r < L)
                     ? *reinterpret_cast<const u32x4_t*>(k + head_off + (size_t)(t0 + r) * D + col)
                     : u32x4_t{0u, 0u, 0u, 0u};
    }
    constexpr int VU = (BLK / 4) * (D / 8);           // (4 keys x 8 d) units of V
    constexpr int VIT = (VU + T::NT - 1) / T::NT;
    u32x4_t vr[VIT][4];
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
        const int u = tid + it * T::NT;
        const int kg = u / (D / 8), dc = u % (D / 8);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = kg * 4 + rr;
            vr[it][rr] = (u < VU && t0 + r < L)
                             ? *reinterpret_cast<const u32x4_t*>(v + head_off + (size_t)(t0 + r) * D + dc * 8)
                             : u32x4_t{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
        const int c = tid + it * T::NT;
        if (c < KCH) {
            const int r = c / (D / 8), col = (c % (D / 8)) * 8;
            *reinterpret_cast<u32x4_t*>(Ks + r * T::KP + col) = kr[it];
        }
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
        const int u = tid + it * T::NT;
        if (u < VU) {
            const int kg = u / (D / 8), dc = u % (D / 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int sh = (e & 1) ? 16 : 0;
                const uint32_t b0 = (vr[it][0][e / 2] >> sh) & 0xFFFFu;
                const uint32_t b1 = (vr[it][1][e / 2] >> sh) & 0xFFFFu;
                const uint32_t b2 = (vr[it][2][e / 2] >> sh) & 0xFFFFu;
                const uint32_t b3 = (vr[it][3][e / 2] >> sh) & 0xFFFFu;
                const u32x2_t w2 = {b0 | (b1 << 16), b2 | (b3 << 16)};
                *reinterpret_cast<u32x2_t*>(Vt + (dc * 8 + e) * T::VP + kg * 4) = w2;
            }
        }
    }
}

template <int D, int BLK, bool DENSE>
__global__ void __launch_bounds__(4 * BLK) attn_bf16_kernel(AttnArgs a) {
    using T = Bf16Tile<D, BLK>;
    __shared__ __align__(16) u16 Ks[BLK * T::KP];
    __shared__ __align__(16) u16 Vt[D * T::VP];
    __shared__ __align__(16) float qb_s[D];
    __shared__ int sel_list[BLK];
    __shared__ unsigned char flag_s[BLK];  // 0 approximate, 1 exact, 2 past N
    __shared__ int misc_s[2];

    const u16* __restrict__ qg = static_cast<const u16*>(a.q);
    const u16* __restrict__ kg = static_cast<const u16*>(a.k);
    const u16* __restrict__ vg = static_cast<const u16*>(a.v);
    u16* __restrict__ og = static_cast<u16*>(a.out);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int H = a.H, L = a.L, N = a.N;

    int dense_item = -1;
    if (DENSE) {
        // XCD-contiguous: XCD x runs items [x*per, (x+1)*per) in order.
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
        const int q0 = i * BLK;
        const size_t head_off = (size_t)h * L * D;

        bf16x8_t qf[T::NS];
        {
            const int row = q0 + wave * 16 + l16;
            const u16* src = qg + head_off + (size_t)row * D + g * 8;
#pragma unroll
            for (int s = 0; s < T::NS; ++s)
                qf[s] = as_bf16x8(row < L ? *reinterpret_cast<const u32x4_t*>(src + s * 32)
                                          : u32x4_t{0u, 0u, 0u, 0u});
        }
        float tau_i = 0.0f;
        if (!DENSE) {
            for (int t = tid; t < D; t += T::NT) qb_s[t] = a.qbar[(size_t)item * D + t];
            tau_i = a.tau[item];
        }

        float m_run = -INFINITY, l_run = 0.0f;
        f32x4_t o[T::NDT];
#pragma unroll
        for (int dt = 0; dt < T::NDT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        const int nch = (N + BLK - 1) / BLK;
        for (int ch = 0; ch < nch; ++ch) {
            const int j0 = ch * BLK;
            const int nj = min(BLK, N - j0);
            int nex = nj;
            if (!DENSE) {
                __syncthreads();
                // Route this chunk of pooled keys and stage it for the
                // approximate path: Kbar rows (bf16) -> Ks, Vsum (bf16) -> Vt.
                {
                    const int jj = tid >> 2, qq = tid & 3;
                    const int jc = min(j0 + jj, N - 1);
                    const bool valid = jj < nj;
                    float kv[D / 4];
                    load_kbar_quarter<D>(a.kbar + ((size_t)h * N + jc) * D, qq, kv);
                    const float s = proxy_from_quarter<D>(qb_s, kv, qq, a.c);
                    const bool sel = valid && (s > tau_i);
                    if (qq == 0) flag_s[jj] = sel ? 1 : (valid ? 0 : 2);
                    u16* kd = Ks + jj * T::KP + qq * (D / 4);
#pragma unroll
                    for (int e = 0; e < D / 4; e += 2)
                        *reinterpret_cast<uint32_t*>(kd + e) = valid ? pack_bf16x2(kv[e], kv[e + 1]) : 0u;
                    float vv[D / 4];
                    load_kbar_quarter<D>(a.vsum + ((size_t)h * N + jc) * D, qq, vv);
#pragma unroll
                    for (int e = 0; e < D / 4; ++e)
                        Vt[(qq * (D / 4) + e) * T::VP + jj] = valid ? f32_to_bf16_bits(vv[e]) : u16(0);
                }
                __syncthreads();
                if (wave == 0) {
                    int base = 0;
#pragma unroll
                    for (int hh = 0; hh < BLK / 64; ++hh) {
                        const int jj = hh * 64 + lane;
                        const bool sel = flag_s[jj] == 1;
                        const uint64_t msk = __ballot(sel);
                        const int pos = base + __popcll(msk & ((1ull << lane) - 1ull));
                        if (sel) sel_list[pos] = j0 + jj;
                        base += __popcll(msk);
                        if (a.sel_dbg) {
                            const int w0 = (j0 + hh * 64) >> 5;
                            uint32_t* dst = a.sel_dbg + (size_t)item * a.W;
                            if (lane == 0 && w0 < a.W) dst[w0] = static_cast<uint32_t>(msk);
                            if (lane == 1 && w0 + 1 < a.W) dst[w0 + 1] = static_cast<uint32_t>(msk >> 32);
                        }
                    }
                    if (lane == 0) misc_s[1] = base;
                }
                __syncthreads();
                nex = misc_s[1];
                if (nex < nj) {
                    // Approximate path: S~^T = Kbar_chunk Q_i^T (Eq. (11)),
                    // weights n_j (Eq. (9)), summed values (Eq. (10)).
                    f32x4_t sacc[T::NKT];
                    scores_t<D, BLK>(Ks, qf, sacc, l16, g);
                    float x[T::NKT][4], w[T::NKT][4];
#pragma unroll
                    for (int kt = 0; kt < T::NKT; ++kt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int jj = kt * 16 + g * 4 + r;
                            x[kt][r] = flag_s[jj] == 0 ? sacc[kt][r] * a.c_log2e : -INFINITY;
                            w[kt][r] = (j0 + jj == N - 1) ? static_cast<float>(a.nlast)
                                                          : static_cast<float>(BLK);
                        }
                    softmax_pv<D, BLK>(x, w, Vt, m_run, l_run, o, l16, g);
                }
            }
            // Exact path over this chunk's selected key blocks (all, if dense).
            for (int e = 0; e < nex; ++e) {
                const int j = DENSE ? j0 + e : sel_list[e];
                __syncthreads();
                stage_kv<D, BLK>(kg, vg, head_off, L, j, Ks, Vt, tid);
                __syncthreads();
                f32x4_t sacc[T::NKT];
                scores_t<D, BLK>(Ks, qf, sacc, l16, g);
                float x[T::NKT][4], w[T::NKT][4];
                const int kvalid = (j == N - 1) ? a.nlast : BLK;
#pragma unroll
                for (int kt = 0; kt < T::NKT; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int jj = kt * 16 + g * 4 + r;
                        x[kt][r] = jj < kvalid ? sacc[kt][r] * a.c_log2e : -INFINITY;
                        w[kt][r] = 1.0f;
                    }
                softmax_pv<D, BLK>(x, w, Vt, m_run, l_run, o, l16, g);
            }
        }

        // out_r = N_r / D_r
        const float lt = wave_sum_xor16_32(l_run);
        const float inv = 1.0f / lt;
        const int row = q0 + wave * 16 + l16;
        if (row < L) {
            u16* dst = og + head_off + (size_t)row * D + g * 4;
#pragma unroll
            for (int dt = 0; dt < T::NDT; ++dt) {
                const u32x2_t pk = {pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv),
                                    pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv)};
                *reinterpret_cast<u32x2_t*>(dst + dt * 16) = pk;
            }
        }
        if (DENSE) break;
    }
}

// ============================================================================
// attention sweep, fp32 inputs (vector ALU; exact fp32 arithmetic path)
// ============================================================================
// Four consecutive lanes own one query row; lane quarter qq holds d/4 of its
// query and output columns.  The same routing arithmetic as the bf16 kernel.
template <int D, int BLK, bool DENSE>
__global__ void __launch_bounds__(4 * BLK) attn_f32_kernel(AttnArgs a) {
    constexpr int NT = 4 * BLK;
    constexpr int Q4 = D / 4;
    constexpr int KP = D + 4;  // pitch keeps 16-byte alignment
    __shared__ __align__(16) float Kf[BLK * KP];
    __shared__ __align__(16) float Vf[BLK * KP];
    __shared__ __align__(16) float qb_s[D];
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
        float tau_i = 0.0f;
        if (!DENSE) {
            for (int t = tid; t < D; t += NT) qb_s[t] = a.qbar[(size_t)item * D + t];
            tau_i = a.tau[item];
        }
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
                const float p01 = p + __shfl_xor(p, 1);
                const float s = p01 + __shfl_xor(p01, 2);
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
                    const float s = proxy_from_quarter<D>(qb_s, kv, qq, a.c);
                    const bool sel = valid && (s > tau_i);
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
                    for (int hh = 0; hh < BLK / 64; ++hh) {
                        const int jj = hh * 64 + lane;
                        const bool sel = flag_s[jj] == 1;
                        const uint64_t msk = __ballot(sel);
                        const int pos = base + __popcll(msk & ((1ull << lane) - 1ull));
                        if (sel) sel_list[pos] = j0 + jj;
                        base += __popcll(msk);
                        if (a.sel_dbg) {
                            const int w0 = (j0 + hh * 64) >> 5;
                            uint32_t* dst = a.sel_dbg + (size_t)item * a.W;
                            if (lane == 0 && w0 < a.W) dst[w0] = static_cast<uint32_t>(msk);
                            if (lane == 1 && w0 + 1 < a.W) dst[w0 + 1] = static_cast<uint32_t>(msk >> 32);
                        }
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

// ============================================================================
// launchers
// ============================================================================
namespace {

int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}

template <typename K>
int persistent_grid(K kernel, int threads) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    return device_cus() * per_cu;
}

template <int D, int BLK>
hipError_t pool_t(const void* q, const void* k, const void* v, int bf16, int H, int L, int N,
                  float* qbar, float* kbar, float* vsum, hipStream_t s) {
    dim3 grid(H * N), block(256);
    if (bf16)
        hipLaunchKernelGGL((pool_kernel<u16, D, BLK>), grid, block, 0, s, static_cast<const u16*>(q),
                           static_cast<const u16*>(k), static_cast<const u16*>(v), L, N, qbar, kbar, vsum);
    else
        hipLaunchKernelGGL((pool_kernel<float, D, BLK>), grid, block, 0, s, static_cast<const float*>(q),
                           static_cast<const float*>(k), static_cast<const float*>(v), L, N, qbar, kbar,
                           vsum);
    return hipGetLastError();
}

template <int D, int BLK, bool DENSE>
hipError_t attn_t(const AttnArgs& a, int bf16, hipStream_t s) {
    const int threads = 4 * BLK;
    int grid;
    if (bf16) {
        auto kern = attn_bf16_kernel<D, BLK, DENSE>;
        grid = DENSE ? 8 * ((a.H * a.N + 7) / 8) : persistent_grid(kern, threads);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, s, a);
    } else {
        auto kern = attn_f32_kernel<D, BLK, DENSE>;
        grid = DENSE ? 8 * ((a.H * a.N + 7) / 8) : persistent_grid(kern, threads);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const void* q, const void* k, const void* v, int bf16, int H, int L, int d,
                       int B, float* qbar, float* kbar, float* vsum, hipStream_t s) {
    const int N = (L + B - 1) / B;
    if (d == 64 && B == 64) return pool_t<64, 64>(q, k, v, bf16, H, L, N, qbar, kbar, vsum, s);
    if (d == 64 && B == 128) return pool_t<64, 128>(q, k, v, bf16, H, L, N, qbar, kbar, vsum, s);
    if (d == 128 && B == 64) return pool_t<128, 64>(q, k, v, bf16, H, L, N, qbar, kbar, vsum, s);
    if (d == 128 && B == 128) return pool_t<128, 128>(q, k, v, bf16, H, L, N, qbar, kbar, vsum, s);
    return hipErrorInvalidValue;
}

hipError_t launch_route(const float* qbar, const float* kbar, int H, int N, int d, float c,
                        float beta, float* tau, int32_t* kept, int* queues, hipStream_t s) {
    const size_t shm = sizeof(float) * (size_t)N;
    dim3 grid(H * N), block(256);
    if (d == 64)
        hipLaunchKernelGGL(route_kernel<64>, grid, block, shm, s, qbar, kbar, N, c, beta, tau, kept, queues);
    else if (d == 128)
        hipLaunchKernelGGL(route_kernel<128>, grid, block, shm, s, qbar, kbar, N, c, beta, tau, kept, queues);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_reset_counters(int* queues, hipStream_t s) {
    hipLaunchKernelGGL(reset_counters_kernel, dim3(1), dim3(64), 0, s, queues);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, int bf16, int d, int B, bool dense, hipStream_t s) {
    if (d == 64 && B == 64) return dense ? attn_t<64, 64, true>(a, bf16, s) : attn_t<64, 64, false>(a, bf16, s);
    if (d == 64 && B == 128) return dense ? attn_t<64, 128, true>(a, bf16, s) : attn_t<64, 128, false>(a, bf16, s);
    if (d == 128 && B == 64) return dense ? attn_t<128, 64, true>(a, bf16, s) : attn_t<128, 64, false>(a, bf16, s);
    if (d == 128 && B == 128) return dense ? attn_t<128, 128, true>(a, bf16, s) : attn_t<128, 128, false>(a, bf16, s);
    return hipErrorInvalidValue;
}

}  // namespace sol
