// sol_sweep.hip -- the fused Sol-Attn sweep for bf16 inputs on gfx950.
//
// One workgroup owns one query block of BLK rows at a time; wave w owns the
// 32 rows 32w .. 32w+31 (two 16-row MFMA tiles), so each K / V fragment read
// from LDS feeds two v_mfma_f32_16x16x32_bf16.
//
// Per query block i of head h ("Sol-Attn" visual explainer, "The complete
// idea in one pass", Eq. (4), Eq. (9), Eq. (10), Eq. (11)):
//   1. routing, on chip: the proxy scores s_ij of all N pooled keys are
//      recomputed chunk by chunk with the routing kernel's own arithmetic and
//      compared with tau_i; the decisions become an N-bit mask in LDS and a
//      tile list: one approximate tile per chunk of BLK pooled keys that has
//      an unselected block, then one exact tile per selected key block.
//      Scores are never written to memory.
//   2. the tile loop: every tile is BLK keys (pooled keys, or the tokens of a
//      key block) and BLK values (summed values, or the tokens' values),
//      staged in LDS as K [key][d] and V^T [d][key].  Scores are formed
//      transposed, S^T = K Q^T, so each lane holds one query row per 16-row
//      tile and 4 keys per 16-key tile, and the softmax weights feed
//      O^T += V^T P^T from registers.  Approximate tiles weight each pooled
//      key by n_j tokens in the denominator (Eq. (9)) and use summed values
//      (Eq. (10)); selected columns of an approximate tile and padded keys of
//      the last block are masked.  One running max / denominator /
//      accumulator serves both paths.
//   3. out = O / l, rounded to bf16.
// Tiles are software-pipelined: the global loads of tile t+1 are in flight
// in registers while tile t is computed from LDS.
//
// Scheduling: persistent workgroups pull query blocks from eight work
// queues, one per XCD (workgroup w runs on XCD w % 8).  Queue x holds, head
// by head, the query blocks [x N / 8, (x+1) N / 8), so the workgroups of one
// XCD work on neighbouring query blocks of the same head at the same time
// and share its L2; an empty queue sends a workgroup on to the next one.
// Every workgroup exits once all eight queues are drained.  Dense mode:
// every key block exact, no routing, one query block per workgroup.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sol_device.h"
#include "sol_launch.h"

namespace sol {

template <int D, int BLK>
struct Sweep {
    static constexpr int NW = BLK / 32;              // waves, 32 query rows each
    static constexpr int NT = 64 * NW;               // threads
    static constexpr int KP = D + 8;                 // K tile pitch (bf16 elements)
    static constexpr int VP = BLK;                   // V^T tile pitch (XOR-swizzled, no padding)
    static constexpr int NKT = BLK / 16;             // 16-key tiles of S^T
    static constexpr int NS = D / 32;                // 32-deep steps over d
    static constexpr int NDT = D / 16;               // 16-wide d tiles of O^T
    static constexpr int NU = BLK / 32;              // 32-key steps of P V
    static constexpr int KPT = (BLK * D / 8) / NT;   // 16-byte K chunks per thread (D/16)
    static constexpr int VPT = ((BLK / 4) * (D / 8)) / NT;  // (4 keys x 8 d) V units per thread
    static_assert(KPT * NT == BLK * D / 8, "K staging must divide evenly");
    static_assert(VPT * NT == (BLK / 4) * (D / 8), "V staging must divide evenly");
    static constexpr int KEYS_PER_PASS = NT / 4;     // routing: four lanes per pooled key
};

constexpr uint32_t kApprox = 0x80000000u;  // tile-list flag: approximate chunk

// V^T tiles keep 4-key (8-byte) groups; group k of row d is stored at
// position k ^ vt_swz(d).  With a pitch of BLK keys this makes both the
// transposing stores (16 lanes on 16 rows d = 8 dc + e) and the P V operand
// reads (16 lanes on 16 consecutive rows) hit 32 distinct LDS banks.
__device__ __forceinline__ int vt_swz(int d) { return (d & 15) ^ ((d >> 3) & 15); }

// Keep bits 0, 4, 8, ..., 60 of m and pack them into bits 0..15.
__device__ __forceinline__ uint32_t every_fourth_bit(uint64_t m) {
    uint64_t x = m & 0x1111111111111111ull;
    x = (x | (x >> 3)) & 0x0303030303030303ull;
    x = (x | (x >> 6)) & 0x000F000F000F000Full;
    x = (x | (x >> 12)) & 0x000000FF000000FFull;
    x = (x | (x >> 24)) & 0xFFFFull;
    return static_cast<uint32_t>(x);
}

template <int D, int BLK>
struct TileRegs {
    u32x4_t k[Sweep<D, BLK>::KPT];
    u32x4_t v[Sweep<D, BLK>::VPT][4];
};

// Issue the global loads of one tile (BLK rows of K-like and V-like data,
// row-major bf16 with row stride D); rows at or past `nvalid` read as 0.
template <int D, int BLK>
__device__ __forceinline__ void tile_load(TileRegs<D, BLK>& tr, const u16* __restrict__ kp,
                                          const u16* __restrict__ vp, int nvalid, int tid) {
    using S = Sweep<D, BLK>;
#pragma unroll
    for (int it = 0; it < S::KPT; ++it) {
        const int c = tid + it * S::NT;
        const int r = c / (D / 8), col = (c % (D / 8)) * 8;
        tr.k[it] = r < nvalid ? *reinterpret_cast<const u32x4_t*>(kp + (size_t)r * D + col)
                              : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < S::VPT; ++it) {
        const int u = tid + it * S::NT;
        const int kg = u / (D / 8), dc = u % (D / 8);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = kg * 4 + rr;
            tr.v[it][rr] = r < nvalid ? *reinterpret_cast<const u32x4_t*>(vp + (size_t)r * D + dc * 8)
                                      : u32x4_t{0u, 0u, 0u, 0u};
        }
    }
}

// Write a loaded tile to LDS: K row-major, V transposed (4 keys per 8-byte write).
template <int D, int BLK>
__device__ __forceinline__ void tile_store(const TileRegs<D, BLK>& tr, u16* Ks, u16* Vt, int tid) {
    using S = Sweep<D, BLK>;
#pragma unroll
    for (int it = 0; it < S::KPT; ++it) {
        const int c = tid + it * S::NT;
        const int r = c / (D / 8), col = (c % (D / 8)) * 8;
        *reinterpret_cast<u32x4_t*>(Ks + r * S::KP + col) = tr.k[it];
    }
#pragma unroll
    for (int it = 0; it < S::VPT; ++it) {
        const int u = tid + it * S::NT;
        const int kg = u / (D / 8), dc = u % (D / 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // element e of four key rows -> {k0 | k1 << 16, k2 | k3 << 16}
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            const u32x2_t w2 = {__builtin_amdgcn_perm(tr.v[it][1][e / 2], tr.v[it][0][e / 2], sel),
                                __builtin_amdgcn_perm(tr.v[it][3][e / 2], tr.v[it][2][e / 2], sel)};
            const int d = dc * 8 + e;
            *reinterpret_cast<u32x2_t*>(Vt + d * S::VP + ((kg ^ vt_swz(d)) << 2)) = w2;
        }
    }
}

template <int D, int BLK, bool DENSE>
__global__ void __launch_bounds__(2 * BLK) sweep_bf16_kernel(AttnArgs a) {
    using S = Sweep<D, BLK>;
    __shared__ __align__(16) u16 Ks[BLK * S::KP];
    __shared__ __align__(16) u16 Vt[D * S::VP];
    __shared__ __align__(16) float qb_s[D];
    __shared__ int misc_s[2];
    extern __shared__ __align__(16) uint32_t dyn[];  // selection bits, then the tile list

    const u16* __restrict__ qg = static_cast<const u16*>(a.q);
    const u16* __restrict__ kg = static_cast<const u16*>(a.k);
    const u16* __restrict__ vg = static_cast<const u16*>(a.v);
    u16* __restrict__ og = static_cast<u16*>(a.out);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int H = a.H, L = a.L, N = a.N;
    const int NC = (N + BLK - 1) / BLK;
    const int nwords = (N + 31) / 32;
    uint32_t* selbits = dyn;                 // N bits (1 = exact)
    uint32_t* tiles = dyn + nwords;          // up to NC + N entries

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
        const int q0 = i * BLK;
        const size_t head_off = (size_t)h * L * D;

        int T;
        if (DENSE) {
            T = N;
        } else {
            // ---- 1. routing on chip -------------------------------------
            for (int t = tid; t < D; t += S::NT) qb_s[t] = a.qbar[(size_t)item * D + t];
            const float tau_i = a.tau[item];
            __syncthreads();
            {
                const int jj = tid >> 2, qq = tid & 3;
                const size_t kb_head = (size_t)h * N * D;
                for (int j0 = 0; j0 < N; j0 += S::KEYS_PER_PASS) {
                    const int j = j0 + jj;
                    float kv[D / 4];
                    load_kbar_quarter<D>(a.kbar + kb_head + (size_t)min(j, N - 1) * D, qq, kv);
                    const float s = proxy_from_quarter<D>(qb_s, kv, qq, a.c);
                    const bool sel = j < N && s > tau_i;
                    const uint32_t bits = every_fourth_bit(__ballot(sel));  // 16 keys of this wave
                    const int kb = j0 + wave * 16;                          // first key of the wave
                    if (lane == 0 && kb < N) {
                        // 16-bit aligned field of the mask
                        reinterpret_cast<uint16_t*>(selbits)[kb >> 4] = static_cast<uint16_t>(bits);
                    }
                }
            }
            __syncthreads();
            if (wave == 0) {
                // approximate chunks that hold at least one unselected block
                int nt = 0;
                for (int c0 = 0; c0 < NC; c0 += 64) {
                    const int c = c0 + lane;
                    bool need = false;
                    if (c < NC) {
                        const int lo = c * BLK, cnt = min(BLK, N - lo);
                        int ones = 0;
#pragma unroll
                        for (int w32 = 0; w32 < BLK / 32; ++w32) {
                            const int bit0 = lo + 32 * w32;
                            if (bit0 < N) {
                                uint32_t wd = selbits[bit0 >> 5];
                                const int valid = min(32, N - bit0);
                                if (valid < 32) wd &= (1u << valid) - 1u;
                                ones += __popc(wd);
                            }
                        }
                        need = ones < cnt;
                    }
                    const uint64_t m = __ballot(need);
                    if (need) tiles[nt + __popcll(m & ((1ull << lane) - 1ull))] = kApprox | c;
                    nt += __popcll(m);
                }
                // exact tiles, ascending key block
                for (int j0 = 0; j0 < N; j0 += 64) {
                    const int j = j0 + lane;
                    const bool sel = j < N && ((selbits[j >> 5] >> (j & 31)) & 1u);
                    const uint64_t m = __ballot(sel);
                    if (sel) tiles[nt + __popcll(m & ((1ull << lane) - 1ull))] = j;
                    nt += __popcll(m);
                }
                if (lane == 0) misc_s[1] = nt;
                if (a.sel_dbg) {
                    uint32_t* dst = a.sel_dbg + (size_t)item * a.W;
                    for (int w = lane; w < nwords; w += 64) {
                        uint32_t wd = selbits[w];
                        const int valid = N - 32 * w;
                        if (valid < 32) wd &= (1u << valid) - 1u;
                        dst[w] = wd;
                    }
                }
            }
            __syncthreads();
            T = misc_s[1];
        }

        // Q fragments (B operand of S^T = K Q^T): rows 32w + 16qt + l16
        bf16x8_t qf[2][S::NS];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const int row = q0 + wave * 32 + qt * 16 + l16;
            const u16* src = qg + head_off + (size_t)row * D + g * 8;
#pragma unroll
            for (int s = 0; s < S::NS; ++s)
                qf[qt][s] = as_bf16x8(row < L ? *reinterpret_cast<const u32x4_t*>(src + s * 32)
                                              : u32x4_t{0u, 0u, 0u, 0u});
        }

        // ---- 2. the tile loop ---------------------------------------------
        float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};
        f32x4_t o[S::NDT][2];
#pragma unroll
        for (int dt = 0; dt < S::NDT; ++dt) o[dt][0] = o[dt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        auto tile_src = [&](int t, const u16*& kp, const u16*& vp, int& nvalid) {
            const uint32_t desc = DENSE ? static_cast<uint32_t>(t) : tiles[t];
            if (desc & kApprox) {
                const int c = static_cast<int>(desc & ~kApprox);
                const size_t off = ((size_t)h * N + (size_t)c * BLK) * D;
                kp = a.kbar_bf + off;
                vp = a.vsum_bf + off;
                nvalid = min(BLK, N - c * BLK);
            } else {
                const int j = static_cast<int>(desc);
                kp = kg + head_off + (size_t)j * BLK * D;
                vp = vg + head_off + (size_t)j * BLK * D;
                nvalid = min(BLK, L - j * BLK);
            }
        };

        TileRegs<D, BLK> tr;
        if (T > 0) {
            const u16 *kp, *vp;
            int nv;
            tile_src(0, kp, vp, nv);
            tile_load<D, BLK>(tr, kp, vp, nv, tid);
        }
        for (int t = 0; t < T; ++t) {
            __syncthreads();  // the previous tile's readers are done with Ks / Vt
            tile_store<D, BLK>(tr, Ks, Vt, tid);
            __syncthreads();
            const uint32_t desc = DENSE ? static_cast<uint32_t>(t) : tiles[t];
            if (t + 1 < T) {
                const u16 *kp, *vp;
                int nv;
                tile_src(t + 1, kp, vp, nv);
                tile_load<D, BLK>(tr, kp, vp, nv, tid);
            }

            // S^T = K Q^T for this wave's 32 query rows
            f32x4_t sacc[S::NKT][2];
#pragma unroll
            for (int kt = 0; kt < S::NKT; ++kt) sacc[kt][0] = sacc[kt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < S::NS; ++s) {
#pragma unroll
                for (int kt = 0; kt < S::NKT; ++kt) {
                    const u32x4_t av =
                        *reinterpret_cast<const u32x4_t*>(Ks + (kt * 16 + l16) * S::KP + s * 32 + g * 8);
                    sacc[kt][0] = mfma16(as_bf16x8(av), qf[0][s], sacc[kt][0]);
                    sacc[kt][1] = mfma16(as_bf16x8(av), qf[1][s], sacc[kt][1]);
                }
            }

            // masks and weights of this tile's BLK columns
            const bool approx = (desc & kApprox) != 0;
            int c0;
            int nvalid;
            uint64_t colsel = 0, colsel_hi = 0;  // approximate tile: columns computed exactly
            if (approx) {
                const int c = static_cast<int>(desc & ~kApprox);
                c0 = c * BLK;
                nvalid = min(BLK, N - c0);
#pragma unroll
                for (int w32 = 0; w32 < 2; ++w32)
                    if (c0 + 32 * w32 < N)
                        colsel |= static_cast<uint64_t>(selbits[(c0 >> 5) + w32]) << (32 * w32);
                if (BLK == 128) {
#pragma unroll
                    for (int w32 = 2; w32 < 4; ++w32)
                        if (c0 + 32 * w32 < N)
                            colsel_hi |= static_cast<uint64_t>(selbits[(c0 >> 5) + w32]) << (32 * (w32 - 2));
                }
            } else {
                c0 = static_cast<int>(desc) * BLK;
                nvalid = min(BLK, L - c0);
            }
            if (approx || nvalid < BLK) {
                // masked columns -> -inf (raw score units; the scale is positive)
#pragma unroll
                for (int kt = 0; kt < S::NKT; ++kt) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int jj = kt * 16 + g * 4 + r;
                        bool valid = jj < nvalid;
                        if (approx) {
                            const uint64_t cs = jj < 64 ? colsel : colsel_hi;
                            valid = valid && !((cs >> (jj & 63)) & 1ull);
                        }
                        if (!valid) sacc[kt][0][r] = sacc[kt][1][r] = -INFINITY;
                    }
                }
            }

            // Online softmax in base 2 with a lazily raised reference max:
            // the reference m only moves when a row's max exceeds it by more
            // than 8 (so every weight stays <= 2^8); any reference cancels in
            // out = O / l.
            const float cl2 = a.c_log2e;
            float mx[2];
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                float v = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < S::NKT; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) v = fmaxf(v, sacc[kt][qt][r]);
                mx[qt] = max4rows(v) * cl2;
            }
            const bool raise = (mx[0] > m_run[0] + 8.0f) || (mx[1] > m_run[1] + 8.0f);
            if (__builtin_amdgcn_ballot_w64(raise) != 0) {
                float alpha[2];
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    const float m_new = fmaxf(m_run[qt], mx[qt]);
                    alpha[qt] = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run[qt] - m_new);
                    m_run[qt] = m_new;
                    l_run[qt] *= alpha[qt];
                }
#pragma unroll
                for (int dt = 0; dt < S::NDT; ++dt) {
                    o[dt][0] *= alpha[0];
                    o[dt][1] *= alpha[1];
                }
            }
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                const float neg_m = m_run[qt] == -INFINITY ? 0.0f : -m_run[qt];
                float psum = 0.0f;
                if (approx) {
                    // Eq. (9): a pooled key stands for n_j tokens
                    const float wlast = static_cast<float>(a.nlast);
                    const float wblk = static_cast<float>(BLK);
                    const int jlast = N - 1 - c0;
#pragma unroll
                    for (int kt = 0; kt < S::NKT; ++kt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][qt][r], cl2, neg_m));
                            sacc[kt][qt][r] = p;
                            psum = __builtin_fmaf((kt * 16 + g * 4 + r == jlast) ? wlast : wblk, p, psum);
                        }
                } else {
#pragma unroll
                    for (int kt = 0; kt < S::NKT; ++kt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][qt][r], cl2, neg_m));
                            sacc[kt][qt][r] = p;
                            psum += p;
                        }
                }
                l_run[qt] += psum;
            }

            // O^T += V^T P^T.  k-index 8g+e of 32-key step u is key 32u + 4g + e
            // (e < 4) or 32u + 16 + 4g + (e - 4): the keys this lane holds.
#pragma unroll
            for (int u = 0; u < S::NU; ++u) {
                u32x4_t pb[2];
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
                    pb[qt] = u32x4_t{pack_bf16x2(sacc[2 * u][qt][0], sacc[2 * u][qt][1]),
                                     pack_bf16x2(sacc[2 * u][qt][2], sacc[2 * u][qt][3]),
                                     pack_bf16x2(sacc[2 * u + 1][qt][0], sacc[2 * u + 1][qt][1]),
                                     pack_bf16x2(sacc[2 * u + 1][qt][2], sacc[2 * u + 1][qt][3])};
#pragma unroll
                for (int dt = 0; dt < S::NDT; ++dt) {
                    const int d = dt * 16 + l16;
                    const u16* vr = Vt + d * S::VP;
                    const int sw = vt_swz(d);
                    const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vr + (((8 * u + g) ^ sw) << 2));
                    const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vr + (((8 * u + 4 + g) ^ sw) << 2));
                    const bf16x8_t av = as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
                    o[dt][0] = mfma16(av, as_bf16x8(pb[0]), o[dt][0]);
                    o[dt][1] = mfma16(av, as_bf16x8(pb[1]), o[dt][1]);
                }
            }
        }

        // ---- 3. out_r = N_r / D_r --------------------------------------------
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const float lt = sum4rows(l_run[qt]);
            const float inv = 1.0f / lt;
            const int row = q0 + wave * 32 + qt * 16 + l16;
            if (row < L) {
                u16* dst = og + head_off + (size_t)row * D + g * 4;
#pragma unroll
                for (int dt = 0; dt < S::NDT; ++dt) {
                    const u32x2_t pk = {pack_bf16x2(o[dt][qt][0] * inv, o[dt][qt][1] * inv),
                                        pack_bf16x2(o[dt][qt][2] * inv, o[dt][qt][3] * inv)};
                    *reinterpret_cast<u32x2_t*>(dst + dt * 16) = pk;
                }
            }
        }
        if (DENSE) break;
    }
}

// ============================================================================
// launcher
// ============================================================================
namespace {

int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}

template <int D, int BLK, bool DENSE>
hipError_t sweep_t(const AttnArgs& a, hipStream_t s) {
    using S = Sweep<D, BLK>;
    auto kern = sweep_bf16_kernel<D, BLK, DENSE>;
    const int NC = (a.N + BLK - 1) / BLK;
    const size_t dyn = DENSE ? 0 : sizeof(uint32_t) * ((size_t)(a.N + 31) / 32 + NC + a.N);
    int grid;
    if (DENSE) {
        grid = 8 * ((a.H * a.N + 7) / 8);
    } else {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, S::NT, dyn) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        grid = device_cus() * per_cu;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(S::NT), dyn, s, a);
    return hipGetLastError();
}

}  // namespace

size_t sweep_dynamic_lds(int N, int B) {
    const int NC = (N + B - 1) / B;
    return sizeof(uint32_t) * ((size_t)(N + 31) / 32 + NC + N);
}

hipError_t launch_sweep_bf16(const AttnArgs& a, int d, int B, bool dense, hipStream_t s) {
    if (d == 64 && B == 64) return dense ? sweep_t<64, 64, true>(a, s) : sweep_t<64, 64, false>(a, s);
    if (d == 64 && B == 128) return dense ? sweep_t<64, 128, true>(a, s) : sweep_t<64, 128, false>(a, s);
    if (d == 128 && B == 64) return dense ? sweep_t<128, 64, true>(a, s) : sweep_t<128, 64, false>(a, s);
    if (d == 128 && B == 128) return dense ? sweep_t<128, 128, true>(a, s) : sweep_t<128, 128, false>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace sol
