// sol_pool_route.hip -- the two stages before the sweep ("Sol-Attn" visual
// explainer, "The complete idea in one pass": pool Q, K and V into blocks;
// computing the thresholds, which its overview places ahead of the stream of
// proxy scores).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sol_device.h"
#include "sol_launch.h"

namespace sol {

// ============================================================================
// pool: block means of Q and K, block sums of V (Eq. (5) and Eq. (10)
// legends).  One workgroup per (head, block), one pass over the block's
// tokens.  Thread t reads 16-byte vectors at column chunk t % CH of rows
// t / CH, t / CH + RG, ...; the RG row-group partial sums are added in a
// fixed order through LDS.  Optionally also writes bf16 copies of kbar and
// vsum, which the sweep's approximate path feeds to the MFMA.
// ============================================================================
template <typename T, int D, int BLK>
__global__ void __launch_bounds__(256) pool_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, int L, int N,
                                                   float* __restrict__ qbar,
                                                   float* __restrict__ kbar,
                                                   float* __restrict__ vsum,
                                                   u16* __restrict__ kbar_bf,
                                                   u16* __restrict__ vsum_bf) {
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
#pragma unroll
    for (int it0 = 0; it0 < IT; it0 += 4) {
        u32x4_t bq[4], bk[4], bv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = rg + (it0 + u) * RG;
            if (it0 + u < IT && r < n) {
                bq[u] = *reinterpret_cast<const u32x4_t*>(q + base + (size_t)r * D);
                bk[u] = *reinterpret_cast<const u32x4_t*>(k + base + (size_t)r * D);
                bv[u] = *reinterpret_cast<const u32x4_t*>(v + base + (size_t)r * D);
            } else {
                bq[u] = bk[u] = bv[u] = u32x4_t{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float xq, xk, xv;
                if constexpr (sizeof(T) == 2) {
                    const int sh = (e & 1) ? 16 : 0;
                    xq = bf16_bits_to_f32(static_cast<u16>(bq[u][e / 2] >> sh));
                    xk = bf16_bits_to_f32(static_cast<u16>(bk[u][e / 2] >> sh));
                    xv = bf16_bits_to_f32(static_cast<u16>(bv[u][e / 2] >> sh));
                } else {
                    xq = __uint_as_float(bq[u][e]);
                    xk = __uint_as_float(bk[u][e]);
                    xv = __uint_as_float(bv[u][e]);
                }
                aq[e] += xq;
                ak[e] += xk;
                av[e] += xv;
            }
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
        if (which == 0) {
            qbar[o] = s * inv_n;
        } else if (which == 1) {
            const float m = s * inv_n;
            kbar[o] = m;
            if (kbar_bf) kbar_bf[o] = f32_to_bf16_bits(m);
        } else {
            vsum[o] = s;
            if (vsum_bf) vsum_bf[o] = f32_to_bf16_bits(s);
        }
    }
}

__global__ void reset_counters_kernel(int* queues) {
    if (threadIdx.x < 8) queues[threadIdx.x] = 0;
}

// bf16 copies of kbar and vsum for sol_sweep callers that bring their own
// pooled tensors; workgroup 0 also clears the sweep's work counters.
__global__ void __launch_bounds__(256) pooled_to_bf16_kernel(const float* __restrict__ kbar,
                                                             const float* __restrict__ vsum,
                                                             size_t n, u16* __restrict__ kbar_bf,
                                                             u16* __restrict__ vsum_bf,
                                                             int* __restrict__ queues) {
    if (blockIdx.x == 0 && threadIdx.x < 8) queues[threadIdx.x] = 0;
    for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (size_t)gridDim.x * 256) {
        kbar_bf[x] = f32_to_bf16_bits(kbar[x]);
        vsum_bf[x] = f32_to_bf16_bits(vsum[x]);
    }
}

// ============================================================================
// route: per (head h, query block i) the proxy row s_i. over all N key
// blocks (Eq. (11) right-hand side), its population mean and standard
// deviation (Eq. (5)), tau_i = mu_i + beta sigma_i and the kept count
// |{j : s_ij > tau_i}| (Eq. (4)).  One workgroup (256 threads) serves R
// consecutive query blocks of one head (R <= 16: one MFMA row tile), so each
// pooled key is read once per R rows; the rows live in dynamic LDS only.
// The decisions leave as bits (one ballot per 64 key blocks), which both
// sweeps read: the routing kernel is the one place s_ij is formed.
// ============================================================================
// Fixed-budget selection, the comparator the abstract contrasts Sol-Attn
// with (every query block keeps the same share of key blocks, the highest
// proxy scores first): each of the
// nr rows keeps its k largest scores, ties to the lower block index.  Wave
// w ranks rows w, w + 4, ... held in LDS: the k-th largest score is found
// exactly by a binary search over order-preserving 32-bit keys (counts from
// ballots), then every larger score is kept, and of the scores equal to it
// the lowest-index ones until k are kept.  tau = that k-th largest score
// (+inf for k = 0); kept = k.
__device__ __forceinline__ uint32_t order_key(float s) {
    const uint32_t b = __float_as_uint(s + 0.0f);  // -0 counts as +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float order_key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// count of keys >= cand in a row: from registers (kr, nch chunks of 64) or LDS
template <bool REG, int MAXC>
__device__ __forceinline__ int count_at_least(const float* row, const uint32_t (&kr)[MAXC], int N,
                                              int nch, int lane, uint32_t cand) {
    int cnt = 0;
    if constexpr (REG) {
#pragma unroll
        for (int c = 0; c < MAXC; ++c)
            if (c < nch) cnt += __popcll(__ballot(kr[c] >= cand));
    } else {
        for (int j0 = 0; j0 < N; j0 += 64) {
            const int j = j0 + lane;
            cnt += __popcll(__ballot(j < N && order_key(row[j]) >= cand));
        }
    }
    return cnt;
}

template <bool REG>
__device__ __forceinline__ void route_rows_topk(const float* rows, int N, int nr, int k, int wave, int lane,
                                uint32_t* sel, int W, float* tau, int32_t* kept) {
    constexpr int MAXC = REG ? 32 : 1;  // keys held in registers: N <= 64 MAXC
    const int nch = (N + 63) / 64;
    for (int r = wave; r < nr; r += 4) {
        const float* row = rows + r * N;
        uint32_t kr[MAXC];  // key of block 64 c + lane (0, never counted, past N)
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int j = 64 * c + lane;
            kr[c] = (REG && c < nch && j < N) ? order_key(row[j]) : 0u;
        }
        uint32_t T = 0;  // largest key with at least k keys >= it
        for (int b = 31; b >= 0; --b) {
            const uint32_t cand = T | (1u << b);
            if (count_at_least<REG, MAXC>(row, kr, N, nch, lane, cand) >= k) T = cand;
        }
        const int above = T == 0xFFFFFFFFu ? 0 : count_at_least<REG, MAXC>(row, kr, N, nch, lane, T + 1u);
        const int need = k - above;  // keys equal to T still to keep
        uint32_t* srow = sel ? sel + (size_t)r * W : nullptr;
        int seen = 0, cnt = 0;
        for (int j0 = 0; j0 < N; j0 += 64) {
            const int j = j0 + lane;
            const uint32_t kj = j < N ? order_key(row[j]) : 0u;
            const uint64_t eq = __ballot(j < N && kj == T);
            const int rank = seen + __popcll(eq & ((1ull << lane) - 1ull));
            const uint64_t m = __ballot(j < N && (kj > T || (kj == T && rank < need)));
            seen += __popcll(eq);
            cnt += __popcll(m);
            const int w0 = j0 >> 5;
            if (srow && lane < 2 && w0 + lane < W) srow[w0 + lane] = static_cast<uint32_t>(m >> (32 * lane));
        }
        if (lane == 0) {
            tau[r] = k > 0 ? order_key_value(T) : INFINITY;
            kept[r] = cnt;
        }
    }
}

template <int D, int R>
__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ qbar,
                                                    const float* __restrict__ kbar, int N,
                                                    int groups_per_head, float c, float beta,
                                                    const float* __restrict__ tau_in,
                                                    float* __restrict__ tau_out,
                                                    int32_t* __restrict__ kept,
                                                    uint32_t* __restrict__ sel, int W,
                                                    int* __restrict__ queues, int topk) {
    extern __shared__ float rows[];  // [R][N]
    const int h = blockIdx.x / groups_per_head;
    const int i0 = (blockIdx.x % groups_per_head) * R;
    const int nr = min(R, N - i0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (queues && blockIdx.x == 0 && tid < 8) queues[tid] = 0;

    // Proxy rows by fp32 MFMA (v_mfma_f32_16x16x4_f32): the workgroup's
    // rows are one 16-row tile (rows past R or N are formed and not kept);
    // wave w takes 16-key tiles w, w + 4, ...  Lane (l16, g) feeds the MFMA
    // its row's (A) and its key's (B) entries d = g D/4 + s at step s, the
    // same order of d on both sides, so the 32 steps contract all of d.  The
    // next key tile's entries load while the current one is multiplied.
    const int l16 = lane & 15, g = lane >> 4;
    constexpr int QD = D / 4;
    float qv[QD];
    {
        const float4* src = reinterpret_cast<const float4*>(
            qbar + ((size_t)h * N + min(i0 + l16, N - 1)) * D + g * QD);
#pragma unroll
        for (int e = 0; e < QD / 4; ++e) {
            const float4 t = src[e];
            qv[4 * e] = t.x; qv[4 * e + 1] = t.y; qv[4 * e + 2] = t.z; qv[4 * e + 3] = t.w;
        }
    }
    const float* kh = kbar + (size_t)h * N * D;
    const int NKT = (N + 15) / 16;
    auto kload = [&](int kt, float (&kv)[QD]) __attribute__((always_inline)) {
        const float4* src = reinterpret_cast<const float4*>(kh + (size_t)min(kt * 16 + l16, N - 1) * D + g * QD);
#pragma unroll
        for (int e = 0; e < QD / 4; ++e) {
            const float4 t = src[e];
            kv[4 * e] = t.x; kv[4 * e + 1] = t.y; kv[4 * e + 2] = t.z; kv[4 * e + 3] = t.w;
        }
    };
    auto score = [&](int kt, const float (&kv)[QD]) __attribute__((always_inline)) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < QD; ++st) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[st], kv[st], acc, 0, 0, 0);
        const int j = kt * 16 + l16;  // lane holds rows 4g .. 4g+3 of key j
#pragma unroll
        for (int x = 0; x < 4; ++x)
            if (4 * g + x < R && j < N) rows[(4 * g + x) * N + j] = acc[x] * c;
    };
    float kva[QD], kvb[QD];
    if (wave < NKT) kload(wave, kva);
#pragma unroll 1
    for (int kt = wave; kt < NKT; kt += 8) {
        if (kt + 4 < NKT) kload(kt + 4, kvb);
        score(kt, kva);
        if (kt + 4 >= NKT) break;
        if (kt + 8 < NKT) kload(kt + 8, kva);
        score(kt + 4, kvb);
    }
    __syncthreads();

    if (topk >= 0) {
        uint32_t* srows = sel ? sel + ((size_t)h * N + i0) * W : nullptr;
        if (N <= 64 * 32)
            route_rows_topk<true>(rows, N, nr, topk, wave, lane, srows, W, tau_out + (size_t)h * N + i0,
                                  kept + (size_t)h * N + i0);
        else
            route_rows_topk<false>(rows, N, nr, topk, wave, lane, srows, W, tau_out + (size_t)h * N + i0,
                                   kept + (size_t)h * N + i0);
        return;
    }
    // statistics: wave w handles rows w, w+4, ... (lane-strided sums in a
    // fixed order, then a butterfly whose result every lane shares)
    for (int r = wave; r < nr; r += 4) {
        const float* row = rows + r * N;
        float part = 0.0f;
        for (int j = lane; j < N; j += 64) part += row[j];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
        const float mu = part / static_cast<float>(N);
        float pv = 0.0f;
        for (int j = lane; j < N; j += 64) {
            const float dlt = row[j] - mu;
            pv = __builtin_fmaf(dlt, dlt, pv);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) pv += __shfl_xor(pv, off);
        const float sigma = sqrtf(fmaxf(pv / static_cast<float>(N), 0.0f));
        float tau;
        if (tau_in) tau = tau_in[(size_t)h * N + i0 + r];  // thresholds given by the caller
        else if (isinf(beta)) tau = beta;                  // -inf: every block exact; +inf: none
        else tau = __builtin_fmaf(beta, sigma, mu);
        // selection bits of the row, 64 blocks per ballot (bit j % 32 of
        // word j / 32 is block j), and their count
        uint32_t* srow = sel ? sel + ((size_t)h * N + i0 + r) * W : nullptr;
        int cnt = 0;
        for (int j0 = 0; j0 < N; j0 += 64) {
            const int j = j0 + lane;
            const uint64_t m = __ballot(j < N && row[j] > tau);
            cnt += __popcll(m);
            const int w0 = j0 >> 5;
            if (srow && lane < 2 && w0 + lane < W) srow[w0 + lane] = static_cast<uint32_t>(m >> (32 * lane));
        }
        if (lane == 0 && !tau_in) {
            tau_out[(size_t)h * N + i0 + r] = tau;
            kept[(size_t)h * N + i0 + r] = cnt;
        }
    }
}

// ============================================================================
// key moments (Eq. (5)): per head the mean of the pooled keys
// mbar = (1/N) sum_j kbar_j and their second moments
// C = (1/N) sum_j kbar_j kbar_j^T, from which the proxy row's population
// mean and variance follow without forming the row:
// mu_i = c qbar_i . mbar and sigma_i^2 = c^2 qbar_i C qbar_i^T - mu_i^2.
// Workgroup (h, bi, bj) forms the 32x32 block (bi, bj) of C (and, for
// bj = 0, 32 entries of mbar), summing over j in a fixed order.  Per head:
// mbar, then C row-major (D + D*D floats).
// ============================================================================
template <int D>
__global__ void __launch_bounds__(256) key_moments_kernel(const float* __restrict__ kbar, int N,
                                                          float* __restrict__ mom) {
    constexpr int NBK = D / 32;
    __shared__ float ka[64][33];
    __shared__ float kb[64][33];
    const int h = blockIdx.x / (NBK * NBK);
    const int bi = (blockIdx.x / NBK) % NBK, bj = blockIdx.x % NBK;
    const int tid = threadIdx.x, a = tid >> 3, b4 = (tid & 7) * 4;
    const float* kh = kbar + (size_t)h * N * D;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float macc = 0.0f;
    for (int j0 = 0; j0 < N; j0 += 64) {
        __syncthreads();
        for (int x = tid; x < 64 * 32; x += 256) {
            const int jj = x >> 5, e = x & 31, j = j0 + jj;
            ka[jj][e] = j < N ? kh[(size_t)j * D + 32 * bi + e] : 0.0f;
            kb[jj][e] = j < N ? kh[(size_t)j * D + 32 * bj + e] : 0.0f;
        }
        __syncthreads();
#pragma unroll 8
        for (int jj = 0; jj < 64; ++jj) {
            const float x = ka[jj][a];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) acc[cc] = __builtin_fmaf(x, kb[jj][b4 + cc], acc[cc]);
            macc += x;
        }
    }
    const float inv = 1.0f / static_cast<float>(N);
    float* mh = mom + (size_t)h * (D + D * D);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) mh[D + (32 * bi + a) * D + 32 * bj + b4 + cc] = acc[cc] * inv;
    if (bj == 0 && b4 == 0) mh[32 * bi + a] = macc * inv;
}

// ============================================================================
// route from the key moments, for rows too long to hold in LDS (N > 1280):
// per (h, i) the threshold tau_i = mu_i + beta sigma_i (Eq. (4)) with mu_i
// and sigma_i from the moments (Eq. (5), above), then one pass that forms
// every s_ij (Eq. (11) right-hand side) exactly as the row-holding route
// does and keeps only the decision s_ij > tau_i, as bits, and their count.
// One workgroup serves 16 query blocks (one MFMA row tile).  With tau_in,
// or beta = +-inf, the thresholds need no moments.
// ============================================================================
template <int D>
__global__ void __launch_bounds__(256) route_moments_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, const float* __restrict__ mom,
    int N, int groups_per_head, float c, float beta, const float* __restrict__ tau_in,
    float* __restrict__ tau_out, int32_t* __restrict__ kept, uint32_t* __restrict__ sel, int W,
    int* __restrict__ queues) {
    constexpr int R = 16;
    extern __shared__ uint16_t bits16[];  // [R][NKT]: the decisions on 16-key tile kt of row r
    __shared__ float qs[R][D + 1];
    __shared__ float tau_s[R];
    const int h = blockIdx.x / groups_per_head;
    const int i0 = (blockIdx.x % groups_per_head) * R;
    const int nr = min(R, N - i0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int NKT = (N + 15) / 16;
    if (queues && blockIdx.x == 0 && tid < 8) queues[tid] = 0;
    for (int x = tid; x < R * D; x += 256) {
        const int r = x / D, e = x % D;
        qs[r][e] = qbar[((size_t)h * N + min(i0 + r, N - 1)) * D + e];
    }
    __syncthreads();

    // thresholds: wave w takes rows 4w .. 4w+3, lane l the columns l + 64 m of
    // v = qbar_r C, then e_r = v . qbar_r and qbar_r . mbar by butterflies
    if (tau_in || isinf(beta)) {
        if (tid < R) tau_s[tid] = tau_in ? tau_in[(size_t)h * N + min(i0 + tid, N - 1)] : beta;
    } else {
        constexpr int CPL = D / 64;
        const float* mh = mom + (size_t)h * (D + D * D);
        float v[4][CPL];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int m = 0; m < CPL; ++m) v[rr][m] = 0.0f;
#pragma unroll 4
        for (int dp = 0; dp < D; ++dp) {
            float crow[CPL];
#pragma unroll
            for (int m = 0; m < CPL; ++m) crow[m] = mh[D + dp * D + lane + 64 * m];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const float qd = qs[4 * wave + rr][dp];
#pragma unroll
                for (int m = 0; m < CPL; ++m) v[rr][m] = __builtin_fmaf(qd, crow[m], v[rr][m]);
            }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = 4 * wave + rr;
            float e = 0.0f, mu = 0.0f;
#pragma unroll
            for (int m = 0; m < CPL; ++m) {
                const int col = lane + 64 * m;
                e = __builtin_fmaf(qs[r][col], v[rr][m], e);
                mu = __builtin_fmaf(qs[r][col], mh[col], mu);
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                e += __shfl_xor(e, off);
                mu += __shfl_xor(mu, off);
            }
            if (lane == 0) {
                const float m_ = c * mu;
                const float var = fmaxf(c * c * e - m_ * m_, 0.0f);
                tau_s[r] = __builtin_fmaf(beta, sqrtf(var), m_);
            }
        }
    }
    __syncthreads();

    // decisions: the proxy scores as the row-holding route forms them (fp32
    // MFMA, the same operands and order), compared as they leave the MFMA
    const int l16 = lane & 15, g = lane >> 4;
    constexpr int QD = D / 4;
    float qv[QD];
#pragma unroll
    for (int e = 0; e < QD; ++e) qv[e] = qs[l16][g * QD + e];
    const float* kh = kbar + (size_t)h * N * D;
    float tr[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) tr[x] = tau_s[4 * g + x];
    auto kload = [&](int kt, float (&kv)[QD]) __attribute__((always_inline)) {
        const float4* src = reinterpret_cast<const float4*>(kh + (size_t)min(kt * 16 + l16, N - 1) * D + g * QD);
#pragma unroll
        for (int e = 0; e < QD / 4; ++e) {
            const float4 t = src[e];
            kv[4 * e] = t.x; kv[4 * e + 1] = t.y; kv[4 * e + 2] = t.z; kv[4 * e + 3] = t.w;
        }
    };
    auto decide = [&](int kt, const float (&kv)[QD]) __attribute__((always_inline)) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < QD; ++st) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[st], kv[st], acc, 0, 0, 0);
        const int j = kt * 16 + l16;  // lane holds rows 4g .. 4g+3 of key j
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const uint64_t m = __ballot(j < N && acc[x] * c > tr[x]);
            // lanes 16 g' .. 16 g' + 15 hold row 4 g' + x
            if (l16 == 0) bits16[(4 * g + x) * NKT + kt] = static_cast<uint16_t>(m >> (16 * g));
        }
    };
    float kva[QD], kvb[QD];
    if (wave < NKT) kload(wave, kva);
#pragma unroll 1
    for (int kt = wave; kt < NKT; kt += 8) {
        if (kt + 4 < NKT) kload(kt + 4, kvb);
        decide(kt, kva);
        if (kt + 4 >= NKT) break;
        if (kt + 8 < NKT) kload(kt + 8, kva);
        decide(kt + 4, kvb);
    }
    __syncthreads();

    // bits out (bit j % 32 of word j / 32) and the counts
    if (sel)
        for (int x = tid; x < nr * W; x += 256) {
            const int r = x / W, w = x % W;
            const uint32_t lo = bits16[r * NKT + 2 * w];
            const uint32_t hi = 2 * w + 1 < NKT ? bits16[r * NKT + 2 * w + 1] : 0u;
            sel[((size_t)h * N + i0 + r) * W + w] = lo | (hi << 16);
        }
    for (int r = wave; r < nr; r += 4) {
        int cnt = 0;
        for (int kt = lane; kt < NKT; kt += 64) cnt += __popc(bits16[r * NKT + kt]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off);
        if (lane == 0 && !tau_in) {
            tau_out[(size_t)h * N + i0 + r] = tau_s[r];
            kept[(size_t)h * N + i0 + r] = cnt;
        }
    }
}

// ============================================================================
// launchers
// ============================================================================
namespace {

template <int D, int BLK>
hipError_t pool_t(const void* q, const void* k, const void* v, int bf16, int H, int L, int N,
                  float* qbar, float* kbar, float* vsum, u16* kbar_bf, u16* vsum_bf, hipStream_t s) {
    dim3 grid(H * N), block(256);
    if (bf16)
        hipLaunchKernelGGL((pool_kernel<u16, D, BLK>), grid, block, 0, s, static_cast<const u16*>(q),
                           static_cast<const u16*>(k), static_cast<const u16*>(v), L, N, qbar, kbar,
                           vsum, kbar_bf, vsum_bf);
    else
        hipLaunchKernelGGL((pool_kernel<float, D, BLK>), grid, block, 0, s,
                           static_cast<const float*>(q), static_cast<const float*>(k),
                           static_cast<const float*>(v), L, N, qbar, kbar, vsum, kbar_bf, vsum_bf);
    return hipGetLastError();
}

template <int D, int R>
hipError_t route_t(const float* qbar, const float* kbar, int H, int N, float c, float beta,
                   const float* tau_in, float* tau, int32_t* kept, uint32_t* sel, int* queues,
                   int topk, hipStream_t s) {
    const int gph = (N + R - 1) / R;
    const size_t shm = sizeof(float) * (size_t)R * N;
    hipLaunchKernelGGL((route_kernel<D, R>), dim3(H * gph), dim3(256), shm, s, qbar, kbar, N, gph, c,
                       beta, tau_in, tau, kept, sel, (N + 31) / 32, queues, topk);
    return hipGetLastError();
}

template <int D>
hipError_t route_moments_t(const float* qbar, const float* kbar, float* mom, int H, int N, float c,
                           float beta, const float* tau_in, float* tau, int32_t* kept, uint32_t* sel,
                           int* queues, hipStream_t s) {
    if (!tau_in && !isinf(beta)) {
        if (!mom) return hipErrorInvalidValue;
        hipLaunchKernelGGL((key_moments_kernel<D>), dim3(H * (D / 32) * (D / 32)), dim3(256), 0, s, kbar, N,
                           mom);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int gph = (N + 15) / 16;
    const size_t shm = sizeof(uint16_t) * 16 * (size_t)((N + 15) / 16);
    hipLaunchKernelGGL((route_moments_kernel<D>), dim3(H * gph), dim3(256), shm, s, qbar, kbar,
                       static_cast<const float*>(mom), N, gph, c, beta, tau_in, tau, kept, sel, (N + 31) / 32,
                       queues);
    return hipGetLastError();
}

template <int D>
hipError_t route_d(const float* qbar, const float* kbar, float* mom, int H, int N, float c, float beta,
                   const float* tau_in, float* tau, int32_t* kept, uint32_t* sel, int* queues,
                   int topk, hipStream_t s) {
    // as many rows per workgroup (at most one 16-row MFMA tile) as 80 KB of
    // LDS holds (two workgroups per CU share its 160 KB); threshold routing
    // with longer rows takes its statistics from the key moments instead
    // and serves 16 rows per workgroup without holding them
    const size_t row_bytes = sizeof(float) * (size_t)N;
    constexpr size_t kLds = 80 * 1024;
    if (topk < 0 && 16 * row_bytes > kLds)
        return route_moments_t<D>(qbar, kbar, mom, H, N, c, beta, tau_in, tau, kept, sel, queues, s);
#define SOL_ROUTE(R) route_t<D, R>(qbar, kbar, H, N, c, beta, tau_in, tau, kept, sel, queues, topk, s)
    if (16 * row_bytes <= kLds) return SOL_ROUTE(16);
    if (8 * row_bytes <= kLds) return SOL_ROUTE(8);
    if (4 * row_bytes <= kLds) return SOL_ROUTE(4);
    if (2 * row_bytes <= kLds) return SOL_ROUTE(2);
    return SOL_ROUTE(1);
#undef SOL_ROUTE
}

}  // namespace

hipError_t launch_pool(const void* q, const void* k, const void* v, int bf16, int H, int L, int d,
                       int B, float* qbar, float* kbar, float* vsum, u16* kbar_bf, u16* vsum_bf,
                       hipStream_t s) {
    const int N = (L + B - 1) / B;
    if (d == 64 && B == 32) return pool_t<64, 32>(q, k, v, bf16, H, L, N, qbar, kbar, vsum, kbar_bf, vsum_bf, s);
    if (d == 128 && B == 32) return pool_t<128, 32>(q, k, v, bf16, H, L, N, qbar, kbar, vsum, kbar_bf, vsum_bf, s);
    if (d == 64 && B == 64) return pool_t<64, 64>(q, k, v, bf16, H, L, N, qbar, kbar, vsum, kbar_bf, vsum_bf, s);
    if (d == 64 && B == 128) return pool_t<64, 128>(q, k, v, bf16, H, L, N, qbar, kbar, vsum, kbar_bf, vsum_bf, s);
    if (d == 128 && B == 64) return pool_t<128, 64>(q, k, v, bf16, H, L, N, qbar, kbar, vsum, kbar_bf, vsum_bf, s);
    if (d == 128 && B == 128) return pool_t<128, 128>(q, k, v, bf16, H, L, N, qbar, kbar, vsum, kbar_bf, vsum_bf, s);
    return hipErrorInvalidValue;
}

hipError_t launch_pooled_to_bf16(const float* kbar, const float* vsum, size_t n, u16* kbar_bf,
                                 u16* vsum_bf, int* queues, hipStream_t s) {
    const size_t blocks = (n + 255) / 256;
    const int grid = static_cast<int>(blocks < 4096 ? (blocks ? blocks : 1) : 4096);
    hipLaunchKernelGGL(pooled_to_bf16_kernel, dim3(grid), dim3(256), 0, s, kbar, vsum, n, kbar_bf,
                       vsum_bf, queues);
    return hipGetLastError();
}

hipError_t launch_reset_counters(int* queues, hipStream_t s) {
    hipLaunchKernelGGL(reset_counters_kernel, dim3(1), dim3(64), 0, s, queues);
    return hipGetLastError();
}

hipError_t launch_route(const float* qbar, const float* kbar, int H, int N, int d, float c,
                        float beta, const float* tau_in, float* tau, int32_t* kept, uint32_t* sel,
                        int* queues, hipStream_t s, int topk, float* mom) {
    if (d == 64) return route_d<64>(qbar, kbar, mom, H, N, c, beta, tau_in, tau, kept, sel, queues, topk, s);
    if (d == 128) return route_d<128>(qbar, kbar, mom, H, N, c, beta, tau_in, tau, kept, sel, queues, topk, s);
    return hipErrorInvalidValue;
}

}  // namespace sol
