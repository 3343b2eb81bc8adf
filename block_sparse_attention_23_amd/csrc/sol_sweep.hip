// sol_sweep.hip -- the fused Sol-Attn sweep for bf16 inputs on gfx950.
//
// A workgroup (4 waves) owns a group of 128 query rows at a time: four
// 32-row query blocks (B = 32), two 64-row blocks (B = 64) or one 128-row
// block (B = 128); the blocks of a group are consecutive or, where the
// selection favours it, spaced by a per-head group stride (group_map below).
// Wave w owns 32 rows of the group (rows 32w .. 32w+31 of consecutive
// blocks) as two 16-row tiles of v_mfma_f32_16x16x32_bf16.
//
// Per workgroup ("Sol-Attn" visual explainer, "The complete idea in one
// pass", Eq. (4), Eq. (9), Eq. (10), Eq. (11)):
//   1. the tile list: the routing kernel's selection bits of the two query
//      blocks (bit j of block i is s_ij > tau_i) are copied to LDS; a tile
//      list follows: one approximate entry per chunk of max(B, 64) pooled
//      keys that holds an unselected block of a query block, then one exact
//      entry per key block that a query block selected (the union, so a key
//      block chosen by several is loaded once; at B = 32, one 64-key tile per
//      two key blocks that the same query blocks selected), each tagged with
//      the query blocks that use it (at B = 32 each wave reads its own
//      block's bits).
//   2. the tile loop over 64-key tiles.  Tiles stream from HBM straight into
//      LDS (direct-to-LDS buffer loads, 16 bytes a lane) into two buffers, so
//      the next tile loads while the current one is computed; the loads are
//      issued right after the barrier that opens a step (the tile-list words
//      are carried one step ahead in scalar registers), by all four waves,
//      or by the two waves of a query block that skips the current tile.
//      K and V rows sit in padded 1 KB LDS blocks (layout below), and each
//      batch of K or V fragment reads is issued before the MFMAs of the
//      batch before it.  Scores are formed
//      transposed, S^T = K Q^T (each lane: one query row per 16-row tile, 4
//      keys per 16-key tile), and O^T += V^T P^T takes V^T through the
//      transposing LDS read (ds_read_b64_tr_b16) and P^T from registers.
//      Approximate tiles weight each pooled key by the n_j tokens it stands
//      for in the denominator (Eq. (9)) and use summed values (Eq. (10));
//      their selected columns, and padded keys of a ragged last block, are
//      masked.  One running max / denominator / accumulator serves both.
//   3. out = O / l, rounded to bf16.
//
// Scheduling: persistent workgroups pull groups from eight work queues, one
// per XCD (workgroup w runs on XCD w % 8).  Queue x holds, head by head, the
// groups [x G / 8, (x+1) G / 8) of the head's G groups, so the workgroups of
// one XCD work on neighbouring rows of the same head at the same time and
// share its L2.  Every workgroup exits once all eight queues
// are drained.  Dense mode: every key block exact, no routing, one group per
// workgroup.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sol_device.h"
#include "sol_launch.h"
#include "sol_tile.h"

namespace sol {

template <int D, int BLK>
struct Sweep : TileLayout<D> {
    static constexpr int QB = 128 / BLK;                // query blocks per workgroup
    static constexpr int TB = BLK < 64 ? 64 : BLK;      // tokens (or pooled keys) per tile-list entry
    static constexpr int SUB = TB / 64;                 // 64-key tiles per entry
    static constexpr int KPT = BLK < 64 ? 64 / BLK : 1;  // key blocks per exact 64-key tile (2 at B = 32)
    // tile-list entry: bit 31 approximate; bits PS .. 30 the query blocks
    // that use it; bits 0 .. PS-1 the chunk or key block index.  Exact
    // entries at B = 32 instead hold two key blocks: j1 in bits 0 .. 12, j2
    // in bits 13 .. 25, bit 26 set when j2 is present (bits PS .. 30: the
    // query blocks that selected both, as in every entry).
    static constexpr int PB = QB < 2 ? 2 : QB;
    static constexpr int PS = 31 - PB;
};

// Query-block groups.  A workgroup item holds QB = 128 / B query blocks of
// one head.  With group stride s, the head's blocks are cut into runs of
// QB s blocks, and group r of a run holds blocks r, r + s, ..., r + (QB-1) s
// of it; the blocks after the last whole run form groups of consecutive
// blocks.  Stride 1 is plain consecutive grouping.  Where each row of a video
// latent's frame spans s query blocks, stride s puts blocks of neighbouring
// rows at the same horizontal position into one group; their selections
// overlap more than those of side-by-side blocks of one row, and the group's
// union tile list is shorter.  The stride is chosen per head from the
// selection bits by group_cost_kernel.
struct GroupMap {
    int blk0, bstep, nqb;  // block b < nqb of the group is blk0 + b * bstep
};

template <int QB>
__device__ __forceinline__ GroupMap group_map(int gi, int N, int st) {
    const int span = QB * st;
    const int full = (N / span) * span;
    const int nfg = full / QB;  // groups inside whole runs
    if (gi < nfg) return GroupMap{(gi / st) * span + gi % st, st, QB};
    const int b0 = full + (gi - nfg) * QB;
    return GroupMap{b0, 1, min(QB, N - b0)};
}

constexpr int kMaxStride = 8;  // candidate group strides 1 .. kMaxStride
constexpr int kCostGroups = 64;  // groups per workgroup of group_cost_kernel

// Grouping cost of a head at a stride: the sum over the head's groups of the
// number of key blocks that any of the group's query blocks selected (the
// exact entries of its union tile list).  Workgroup (h, s, p) sums groups
// p kCostGroups .. (p+1) kCostGroups - 1 of head h at stride s + 1 into
// part[(h kMaxStride + s) P + p], P = ceil(G / kCostGroups); a wave takes
// every fourth of them, its lanes over the selection words.
template <int QB>
__global__ void __launch_bounds__(256) group_cost_kernel(const uint32_t* __restrict__ sel, int N, int W, int P,
                                                         unsigned long long* __restrict__ part) {
    __shared__ unsigned long long wsum[4];
    const int p = blockIdx.x % P, hs = blockIdx.x / P;
    const int h = hs / kMaxStride, st = hs % kMaxStride + 1;
    const int NG = (N + QB - 1) / QB;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint32_t* sh = sel + (size_t)h * N * W;
    unsigned long long cnt = 0;
    const int g1 = min(NG, (p + 1) * kCostGroups);
    // four groups at a time, so that their loads are in flight together
    for (int gb = p * kCostGroups + wave; gb < g1; gb += 16) {
        GroupMap gm[4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
            gm[x] = gb + 4 * x < g1 ? group_map<QB>(gb + 4 * x, N, st) : GroupMap{0, 0, 0};
        for (int w = lane; w < W; w += 64) {
            uint32_t u[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int b = 0; b < QB; ++b)
                    if (b < gm[x].nqb) u[x] |= sh[(size_t)(gm[x].blk0 + b * gm[x].bstep) * W + w];
#pragma unroll
            for (int x = 0; x < 4; ++x) cnt += (unsigned long long)__popc(u[x]);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off);
    if (lane == 0) wsum[wave] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
}

// The group stride of head h = blockIdx.x: the one of least summed cost, the
// smallest on a tie (one wave).
__global__ void __launch_bounds__(64) group_pick_kernel(const unsigned long long* __restrict__ part, int P,
                                                        int* __restrict__ stride) {
    const int h = blockIdx.x, lane = threadIdx.x;
    unsigned long long best = 0;
    int bs = 1;
    for (int s = 0; s < kMaxStride; ++s) {
        unsigned long long c = 0;
        for (int p = lane; p < P; p += 64) c += part[((size_t)h * kMaxStride + s) * P + p];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
        if (s == 0 || c < best) {
            best = c;
            bs = s + 1;
        }
    }
    if (lane == 0) stride[h] = bs;
}

template <int D, int BLK, bool DENSE, bool ROUTE = false>
__global__ void __launch_bounds__(256, 2) sweep_bf16_kernel(AttnArgs a) {
    using S = Sweep<D, BLK>;
    // two tile buffers as four distinct objects, so the compiler can tell
    // that the loads landing in one buffer do not alias reads of the other
    __shared__ __align__(16) u16 K0[S::KSLOT];
    __shared__ __align__(16) u16 V0[S::VSLOT];
    __shared__ __align__(16) u16 K1[S::KSLOT];
    __shared__ __align__(16) u16 V1[S::VSLOT];
    __shared__ int misc_s[2];
    extern __shared__ __align__(16) uint32_t dyn[];  // selection bits per block, then tile list

    const u16* __restrict__ qg = static_cast<const u16*>(a.q);
    const u16* __restrict__ kg = static_cast<const u16*>(a.k);
    const u16* __restrict__ vg = static_cast<const u16*>(a.v);
    u16* __restrict__ og = static_cast<u16*>(a.out);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform within a wave
    const int l16 = lane & 15, g = lane >> 4;
    const int H = a.H, L = a.L, N = a.N;
    const int NC = (N + S::TB - 1) / S::TB;  // approximate chunks
    const int nwords = (N + 31) / 32;
    const int NG = (N + S::QB - 1) / S::QB;  // 128-row groups per head
    uint32_t* selbits = dyn;                 // [QB][nwords]
    uint32_t* tiles = dyn + S::QB * nwords;  // up to NC + ceil(N / KPT) (+ 8 at B = 32) entries
    const int myb = (wave * 32) / BLK;       // this wave's query block within the group
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t dma_base = dma_lane_base<D>(wave_s, lane);
    // when only one query block uses a tile, the other block's two waves
    // load the next tile alone: wave w covers the loads of waves 2 (w & 1)
    // and 2 (w & 1) + 1
    const uint32_t dma_base2 = dma_lane_base<D>(2 * (wave_s & 1), lane);
    // per-lane LDS read offsets (elements); the rest of each read address
    // (16-key tile, 32-deep or 32-key step, d tile, buffer) is an immediate.
    // K: key l16 of a 16-key tile, 16-byte chunk g of a 32-deep step.  V: the
    // transposing read of key 4g + (l16 >> 2) of a 16-key group, columns
    // 8 ((l16 & 3) >> 1) + 4 (l16 & 1) of a 16-wide d tile.
    const int k_lane = S::kbase(l16 % S::NB) + (l16 / S::NB) * D + 8 * g;
    const int k4 = 4 * g + (l16 >> 2), tp = l16 & 3;
    const int v_lane = (k4 % S::NB) * (512 + S::VPAD) + (k4 / S::NB) * D + 8 * (tp >> 1) + 4 * (tp & 1);

    // The tile buffers start zeroed: a direct-to-LDS load of a row past the
    // end of its source is dropped by the buffer range check, so such rows
    // hold zeros or rows of an earlier tile -- finite values in masked
    // columns, whose weights are exactly zero.
    for (int x = tid; x < S::KSLOT / 8; x += S::NT) {
        const u32x4_t z = {0u, 0u, 0u, 0u};
        reinterpret_cast<u32x4_t*>(K0)[x] = z;
        reinterpret_cast<u32x4_t*>(K1)[x] = z;
    }
    for (int x = tid; x < S::VSLOT / 8; x += S::NT) {
        const u32x4_t z = {0u, 0u, 0u, 0u};
        reinterpret_cast<u32x4_t*>(V0)[x] = z;
        reinterpret_cast<u32x4_t*>(V1)[x] = z;
    }
    __syncthreads();  // the zeros land before any tile load is issued

    int dense_item = -1;
    if (DENSE) {
        const int total = H * NG;
        const int per = (total + 7) / 8;
        const int idx = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
        if ((int)(blockIdx.x >> 3) >= per || idx >= total) return;
        dense_item = idx;
    }

    int prev_item = -1;  // (clock records) the item this workgroup finished last
    for (;;) {
        int item;
        if (DENSE) {
            item = dense_item;
        } else {
            __syncthreads();
            if (tid == 0) {
                const int it = a.order ? claim_ordered(a.queues, a.order, H * NG) : claim_item(a.queues, H, NG);
                if (a.trace) {
                    // every wave has finished prev_item (the barrier above)
                    const unsigned long long now = __builtin_amdgcn_s_memrealtime();
                    if (prev_item >= 0) a.trace[3 * (size_t)prev_item + 1] = now;
                    if (it >= 0) {
                        a.trace[3 * (size_t)it] = now;
                        a.trace[3 * (size_t)it + 2] = blockIdx.x;
                    }
                }
                misc_s[0] = it;
            }
            __syncthreads();
            item = __builtin_amdgcn_readfirstlane(misc_s[0]);
            if (item < 0) break;
            prev_item = item;
        }
        const int h = item / NG, gi = item % NG;
        // the head's group stride (group_pick_kernel)
        const int st = (!DENSE && !ROUTE && S::QB > 1 && a.gcost) ? a.gstride[h] : 1;
        const GroupMap gm = group_map<S::QB>(gi, N, st);
        const int nqb = gm.nqb;  // valid query blocks in this group
        // first row of this wave's 32 (rows of query block myb of the group)
        const int r0 = (gm.blk0 + myb * gm.bstep) * BLK + (wave * 32) % BLK;
        const size_t head_off = (size_t)h * L * D;

        int T;
        if (DENSE) {
            T = N;
        } else {
            // ---- 1. the tile list ------------------------------------------
            // selection bits of the group's query blocks: bit j of block i
            // is s_ij > tau_i
            if constexpr (ROUTE) {
                // routed here ("Sol-Attn" visual explainer, Eq. (4) and
                // Eq. (11)): the proxy score of block i and key block j is
                // qbar_i . kbar_j / sqrt(d), the column mean over block i's
                // query tokens of their scores against pooled key j.  It is
                // formed in fp32 from the fp32 pooled vectors (the bf16 MFMA
                // operands of the approximate tiles would move decisions by
                // more than the rounding of an fp32 score) and compared with
                // the block's threshold as each word of 32 key blocks
                // appears; the words live in LDS for this group only.
                float* qs = reinterpret_cast<float*>(K0);  // [QB][D] pooled queries; K0 holds no tile yet
                for (int x = tid; x < S::QB * D; x += S::NT) {
                    const int b = x / D, e = x % D;
                    qs[x] = b < nqb ? a.qbar[((size_t)h * N + gm.blk0 + b * gm.bstep) * D + e] : 0.0f;
                }
                __syncthreads();
                constexpr int DQ = D / 4;                 // a key row is split over 4 lanes
                const int qd = lane & 3, kl = lane >> 2;  // quarter of d, key of 16
                float tc[S::QB];
#pragma unroll
                for (int b = 0; b < S::QB; ++b)
                    tc[b] = b < nqb ? a.tau_cmp[(size_t)h * N + gm.blk0 + b * gm.bstep] : INFINITY;
                const float* kh = a.kbar + (size_t)h * N * D;
                for (int wd = wave; wd < nwords; wd += 4) {
                    uint32_t word[S::QB];
#pragma unroll
                    for (int b = 0; b < S::QB; ++b) word[b] = 0u;
#pragma unroll 1
                    for (int half = 0; half < 2; ++half) {
                        const int j = 32 * wd + 16 * half + kl;
                        const float4* kr = reinterpret_cast<const float4*>(kh + (size_t)min(j, N - 1) * D + qd * DQ);
                        float acc[S::QB];
#pragma unroll
                        for (int b = 0; b < S::QB; ++b) acc[b] = 0.0f;
#pragma unroll
                        for (int e4 = 0; e4 < DQ / 4; ++e4) {
                            const float4 kv = kr[e4];
#pragma unroll
                            for (int b = 0; b < S::QB; ++b) {
                                const float4 qv = *reinterpret_cast<const float4*>(qs + b * D + qd * DQ + 4 * e4);
                                acc[b] = __builtin_fmaf(qv.x, kv.x, acc[b]);
                                acc[b] = __builtin_fmaf(qv.y, kv.y, acc[b]);
                                acc[b] = __builtin_fmaf(qv.z, kv.z, acc[b]);
                                acc[b] = __builtin_fmaf(qv.w, kv.w, acc[b]);
                            }
                        }
#pragma unroll
                        for (int b = 0; b < S::QB; ++b) {
                            acc[b] += __shfl_xor(acc[b], 1);
                            acc[b] += __shfl_xor(acc[b], 2);
                            // bit 4k of m: key 16 half + k of the word
                            const uint64_t m = __ballot(qd == 0 && j < N && acc[b] * a.c > tc[b]);
                            uint32_t v16 = 0;
#pragma unroll
                            for (int k2 = 0; k2 < 16; ++k2) v16 |= (uint32_t)((m >> (4 * k2)) & 1u) << k2;
                            word[b] |= v16 << (16 * half);
                        }
                    }
                    if (lane == 0)
#pragma unroll
                        for (int b = 0; b < S::QB; ++b) selbits[b * nwords + wd] = word[b];
                }
                __syncthreads();
                // kept counts, and the decision bits when asked for
                for (int b = wave; b < nqb; b += 4) {
                    int cnt = 0;
                    for (int w = lane; w < nwords; w += 64) cnt += __popc(selbits[b * nwords + w]);
#pragma unroll
                    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off);
                    if (lane == 0) a.kept_out[(size_t)h * N + gm.blk0 + b * gm.bstep] = cnt;
                }
                if (a.sel_out)
                    for (int t = tid; t < nqb * nwords; t += S::NT) {
                        const int b = t / nwords, w = t % nwords;
                        a.sel_out[((size_t)h * N + gm.blk0 + b * gm.bstep) * a.W + w] = selbits[t];
                    }
            } else {
                // written by the routing kernel
                for (int t = tid; t < S::QB * nwords; t += S::NT) {
                    const int b = t / nwords, w = t % nwords;
                    selbits[t] = b < nqb ? a.sel[((size_t)h * N + gm.blk0 + b * gm.bstep) * a.W + w] : 0u;
                }
            }
            __syncthreads();
            if (wave == 0) {
                const uint32_t all_blocks = (1u << nqb) - 1u;  // selection masks are 1 .. all_blocks
                int nt = 0;
                // approximate chunks that hold an unselected block of a query
                // block (none when the unselected blocks are dropped)
                for (int c0 = 0; c0 < (a.drop_approx ? 0 : NC); c0 += 64) {
                    const int c = c0 + lane;
                    uint32_t part = 0;
                    if (c < NC) {
                        const int lo = c * S::TB, cnt = min(S::TB, N - lo);
                        for (int b = 0; b < nqb; ++b) {
                            int ones = 0;
#pragma unroll
                            for (int w32 = 0; w32 < S::TB / 32; ++w32) {
                                const int bit0 = lo + 32 * w32;
                                if (bit0 < N) {
                                    uint32_t wd = selbits[b * nwords + (bit0 >> 5)];
                                    const int valid = min(32, N - bit0);
                                    if (valid < 32) wd &= (1u << valid) - 1u;
                                    ones += __popc(wd);
                                }
                            }
                            if (ones < cnt) part |= 1u << b;
                        }
                    }
                    const uint64_t m = __ballot(part != 0);
                    if (part) tiles[nt + __popcll(m & ((1ull << lane) - 1ull))] = kApprox | (part << S::PS) | c;
                    nt += __popcll(m);
                }
                // exact key blocks, ascending
                if constexpr (S::KPT == 1) {
                    for (int j0 = 0; j0 < N; j0 += 64) {
                        const int j = j0 + lane;
                        uint32_t part = 0;  // rows of blocks past the group's last are zero
                        if (j < N)
#pragma unroll
                            for (int b = 0; b < S::QB; ++b)
                                part |= ((selbits[b * nwords + (j >> 5)] >> (j & 31)) & 1u) << b;
                        const uint64_t m = __ballot(part != 0);
                        if (part) tiles[nt + __popcll(m & ((1ull << lane) - 1ull))] = (part << S::PS) | j;
                        nt += __popcll(m);
                    }
                } else {
                    // B = 32: key blocks that the same query blocks select
                    // share a 64-key tile, so both halves of a tile serve the
                    // same waves.  Key blocks are taken in ascending order;
                    // lane m (1 <= m <= all_blocks) keeps the state of
                    // selection mask m: `pend`, a block of mask m still
                    // waiting for a partner (-1: none).  In a chunk of 64
                    // blocks, those of mask m pair up in order, the first with
                    // the pending one; an odd last one waits.  The chunk's
                    // entries go out mask by mask, ascending.  Blocks left
                    // waiting at the end get a tile of their own.
                    int pend = -1;
                    // the selection words of the chunk from j0: lane l < 2 QB
                    // reads word j0 / 32 + (l & 1) of row l / 2 (clamped to the
                    // last word; bits of blocks past N are cleared below)
                    auto chunk_word = [&](int j0) {
                        const int w = min((j0 >> 5) + (lane & 1), nwords - 1);
                        return selbits[((lane >> 1) & (S::QB - 1)) * nwords + w];
                    };
                    uint32_t wnext = chunk_word(0);
                    for (int j0 = 0; j0 < N; j0 += 64) {
                        // the lane index, opaque here so that the lane masks
                        // below stay in this loop instead of holding registers
                        // through the sweep
                        int ln = lane;
                        asm volatile("" : "+v"(ln));
                        const bool mlane = ln >= 1 && ln <= (int)all_blocks;
                        const uint64_t below = (1ull << ln) - 1ull;     // lanes before this one
                        const uint64_t above = ~((2ull << ln) - 1ull);  // lanes after it
                        const int j = j0 + ln;
                        const uint32_t wcur = wnext;
                        wnext = chunk_word(j0 + 64);  // next chunk's, read while this one is built
                        // row b's bits of the chunk's 64 blocks, lane k for block j0 + k
                        const uint64_t valid = N - j0 >= 64 ? ~0ull : (1ull << (N - j0)) - 1ull;
                        uint64_t rowb[S::QB], nz = 0;
#pragma unroll
                        for (int b = 0; b < S::QB; ++b) {
                            const uint32_t lo = __builtin_amdgcn_readlane(wcur, 2 * b);
                            const uint32_t hi = __builtin_amdgcn_readlane(wcur, 2 * b + 1);
                            rowb[b] = (((uint64_t)hi << 32) | lo) & valid;
                            nz |= rowb[b];
                        }
                        uint32_t part = 0;  // the query blocks that selected block j
                        // lanes of mask m = lane (1 <= m <= all_blocks)
                        uint64_t mine = nz;
#pragma unroll
                        for (int b = 0; b < S::QB; ++b) {
                            part |= (uint32_t)((rowb[b] >> ln) & 1u) << b;
                            mine &= ((ln >> b) & 1) ? rowb[b] : ~rowb[b];
                        }
                        if (!mlane) mine = 0;
                        // per mask (lane m): blocks in the chunk, the pending
                        // block's partner taken, entries emitted, next pending
                        const int c_m = __popcll(mine);
                        const int q_m = (c_m > 0 && pend >= 0) ? 1 : 0;
                        const int n_m = c_m > 0 ? q_m + ((c_m - q_m) >> 1) : 0;
                        // inclusive prefix over each row of 16 lanes (DPP row
                        // shifts by 1, 2, 4, 8; lanes shifted in from outside
                        // the row read 0)
                        int incl = n_m;
                        incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xf, 0xf, true);
                        incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xf, 0xf, true);
                        incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xf, 0xf, true);
                        incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xf, 0xf, true);
                        // from mask lane `part`: the lanes of this block's mask,
                        // the mask's first entry in the chunk and its pending
                        // block (lane 0 holds no mask: zeros for part = 0)
                        const uint64_t own = ((uint64_t)(uint32_t)__shfl((int)(uint32_t)(mine >> 32), (int)part) << 32) |
                                             (uint32_t)__shfl((int)(uint32_t)mine, (int)part);
                        const int fp = __shfl(((incl - n_m) << 16) | (pend & 0xffff), (int)part);
                        const int off = fp >> 16;
                        const int p = (int16_t)(fp & 0xffff);
                        if (part) {
                            const int q = p >= 0 ? 1 : 0;
                            const int r = __popcll(own & below);  // rank among the blocks of its mask
                            const uint32_t tag = part << S::PS;
                            if (q && r == 0) {
                                tiles[nt + off] = (uint32_t)p | ((uint32_t)j << 13) | (1u << 26) | tag;
                            } else if (((r - q) & 1) == 0 && (own & above) != 0) {
                                // j1 of a pair: j2 is the next block of the same mask
                                const int j2 = j0 + __builtin_ctzll(own & above);
                                tiles[nt + off + q + ((r - q) >> 1)] =
                                    (uint32_t)j | ((uint32_t)j2 << 13) | (1u << 26) | tag;
                            }
                        }
                        nt += __builtin_amdgcn_readlane(incl, 15);
                        if (c_m > 0) pend = ((c_m - q_m) & 1) ? j0 + 63 - __builtin_clzll(mine) : -1;
                    }
                    // blocks still waiting: a tile each (no second half)
                    const uint64_t wb = __ballot(lane >= 1 && lane <= (int)all_blocks && pend >= 0);
                    if (lane >= 1 && lane <= (int)all_blocks && pend >= 0)
                        tiles[nt + __popcll(wb & ((1ull << lane) - 1ull))] = (uint32_t)pend | ((uint32_t)lane << S::PS);
                    nt += __popcll(wb);
                }
                if (lane == 0) misc_s[1] = nt;
            }
            __syncthreads();
            T = __builtin_amdgcn_readfirstlane(misc_s[1]);
        }

        // Q fragments (B operand of S^T = K Q^T): rows r0 + 16qt + l16
        bf16x8_t qf[2][S::NS];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const int row = r0 + qt * 16 + l16;
            const u16* src = qg + head_off + (size_t)row * D + g * 8;
#pragma unroll
            for (int s = 0; s < S::NS; ++s)
                qf[qt][s] = as_bf16x8(row < L ? *reinterpret_cast<const u32x4_t*>(src + s * 32)
                                              : u32x4_t{0u, 0u, 0u, 0u});
        }

        // ---- 2. the tile loop ---------------------------------------------
        // o[0..NDT-1]: O^T tiles; o[NDT]: the softmax denominator, formed by
        // the MFMA from a weight row (row 0 of an extra 16-row V^T tile holds
        // each key's weight: 1 per token, n_j per pooled key -- Eq. (9)), so
        // numerator and denominator use the same bf16-rounded weights.
        float m_run[2] = {-INFINITY, -INFINITY};
        f32x4_t o[S::NDT + 1][2];
#pragma unroll
        for (int dt = 0; dt <= S::NDT; ++dt) o[dt][0] = o[dt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // weight-row operands: lanes with l16 == 0 carry row 0 (8 keys each)
        const uint32_t one2 = l16 == 0 ? 0x3F803F80u : 0u;  // bf16 1.0, 1.0
        const uint32_t blk2 = l16 == 0 ? pack_bf16x2(static_cast<float>(BLK), static_cast<float>(BLK)) : 0u;

        const uint32_t all_part = (1u << nqb) - 1u;
        // Tile-list word of 64-key tile t: the raw LDS value, then the word
        // itself, the same for the whole workgroup (kept scalar).
        auto word_raw = [&](int t) -> uint32_t { return DENSE ? 0u : tiles[t / S::SUB]; };
        auto word_of = [&](int t, uint32_t raw) -> uint32_t {
            return DENSE ? ((all_part << S::PS) | (uint32_t)(t / S::SUB))
                         : (uint32_t)__builtin_amdgcn_readfirstlane((int)raw);
        };
        // (approx?, part, row0 of the tile in its source) of tile t; a B = 32
        // pair entry holds two key blocks instead of an index (row0 = 0,
        // unused: its rows come from pair_of)
        auto decode = [&](uint32_t d, int t, bool& approx, uint32_t& part, int& row0) {
            approx = (d & kApprox) != 0;
            part = (d >> S::PS) & ((1u << S::PB) - 1u);
            row0 = (S::KPT == 2 && !approx) ? 0 : (int)(d & ((1u << S::PS) - 1u)) * S::TB + (t % S::SUB) * 64;
        };
        // (B = 32 exact entries) the pair's key blocks
        auto pair_of = [&](uint32_t d, int& j1, int& j2, bool& has2) {
            j1 = (int)(d & 0x1FFFu);
            j2 = (int)((d >> 13) & 0x1FFFu);
            has2 = ((d >> 26) & 1u) != 0;
        };
        // lanes 0-31 load keys 0-31 of a tile and lanes 32-63 keys 32-63
        const bool lo_lanes = lane < 32;
        // resources of tile t and this lane's extra source offset (bytes)
        auto source_of = [&](uint32_t d, int t, uint32_t& extra) {
            bool ap;
            uint32_t pt;
            int row0;
            decode(d, t, ap, pt, row0);
            extra = 0;
            if (S::KPT == 2 && !ap) {
                // a pair: rows 32 j1 + k (k < 32) and 32 j2 + k - 32; an
                // absent j2 points past L, so its loads are dropped
                int j1, j2;
                bool has2;
                pair_of(d, j1, j2, has2);
                const int rb = lo_lanes ? 32 * j1 : (has2 ? 32 * j2 - 32 : L);
                extra = (uint32_t)rb * (2u * D);
                return rows_src<D>(kg + head_off, vg + head_off, L);
            }
            // choose the source before forming its resources (kept scalar)
            const u16* kp = ap ? a.kbar_bf + (size_t)h * N * D : kg + head_off;
            const u16* vp = ap ? a.vsum_bf + (size_t)h * N * D : vg + head_off;
            return tile_src<D>(kp, vp, row0, ap ? N : L);
        };
        // Carried from step to step, so that a step issues its loads right
        // after its barrier with no LDS read first: the words of tiles t and
        // t+1 (scalars).
        uint32_t w_t = 0, w_t1 = 0;

        // compute tile t from (Kt, Vt) while tile t+1 streams into (Kn, Vn)
        auto step = [&](int t, const u16* Kt, const u16* Vt, u16* Kn, u16* Vn, int TS) {
            __builtin_amdgcn_s_waitcnt(0);  // this thread's loads of tile t have landed
            __syncthreads();                // everyone's have; tile t-1 is no longer read
            bool approx;
            uint32_t part;
            int row0;
            decode(w_t, t, approx, part, row0);
            // this wave's query block uses tile t (a B = 32 pair entry carries
            // the query blocks that selected both of its key blocks)
            const bool mine = ((part >> myb) & 1u) != 0u;
            // B = 32 pairs: bit h of halves: this wave's query block selected
            // key block h of the pair; lim_h: keys of half h before L
            uint32_t halves = 3u;
            int lim_h[2] = {0, 0};
            if (S::KPT == 2 && !approx) {
                int j1, j2;
                bool has2;
                pair_of(w_t, j1, j2, has2);
                halves = mine ? (has2 ? 3u : 1u) : 0u;
                lim_h[0] = L - 32 * j1;
                lim_h[1] = L - 32 * j2 + 32;
            }
            if (t + 1 < TS) {  // tile t+1 streams into (Kn, Vn)
                uint32_t extra;
                if constexpr (S::KPT == 2) {
                    const TileSrc nsrc = source_of(w_t1, t + 1, extra);
                    tile_issue<D>(nsrc, Kn, Vn, wave_s, dma_base + extra);
                } else if (S::QB != 2 || part == 3u) {
                    tile_issue<D>(source_of(w_t1, t + 1, extra), Kn, Vn, wave_s, dma_base);
                } else if (!mine) {
                    tile_issue<D, 0, 2 * S::LPT>(source_of(w_t1, t + 1, extra), Kn, Vn, 2 * (wave_s & 1),
                                                      dma_base2);
                }
            }
            const uint32_t raw2 = t + 2 < TS ? word_raw(t + 2) : 0u;
            // move the carried state on to tile t+1
            auto advance = [&]() __attribute__((always_inline)) {
                w_t = w_t1;
                w_t1 = t + 2 < TS ? word_of(t + 2, raw2) : 0u;
            };
            advance();
            if (!mine) return;  // this wave's query block does not use tile t

            // S^T = K Q^T for this wave's 32 query rows, one 32-deep step at a
            // time; the K fragments of step s+1 are read before the MFMAs of
            // step s, so each batch of LDS reads hides behind MFMA work (the
            // compiler's MFMA / LDS interleaving strategy 1 orders them).
            f32x4_t sacc[4][2];
            u32x4_t kfr[2][4];
            auto kread = [&](int st, u32x4_t (&dst)[4]) __attribute__((always_inline)) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
                    dst[kt] = *reinterpret_cast<const u32x4_t*>(Kt + k_lane + kt * (16 / S::NB) * D + 32 * st);
            };
            kread(0, kfr[0]);
#pragma unroll
            for (int st = 0; st < S::NS; ++st) {
                if (st == 0) __builtin_amdgcn_iglp_opt(1);
                if (st + 1 < S::NS) kread(st + 1, kfr[(st + 1) & 1]);
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
                    sacc[kt][0] = mfma16(as_bf16x8(kfr[st & 1][kt]), qf[0][st], st == 0 ? z : sacc[kt][0]);
                    sacc[kt][1] = mfma16(as_bf16x8(kfr[st & 1][kt]), qf[1][st], st == 0 ? z : sacc[kt][1]);
                }
            }

            // column masks: tokens past L (exact), selected or past-N pooled
            // keys (approximate), and at B = 32 the key block of a pair that
            // this wave's query block did not select (exact).  Lane key
            // jj = 16 kt + 4g + r is bit 16 kt + r of colsel >> 4g.
            const int limit = approx ? N : L;
            const bool pair = S::KPT == 2 && !approx;
            if (approx || (pair ? (halves != 3u || lim_h[0] < 32 || lim_h[1] < 64) : row0 + 64 > limit)) {
                uint64_t colsel = 0;
                if (approx) {
                    const uint32_t* sb = selbits + myb * nwords;
                    if (row0 < N) colsel = sb[row0 >> 5];
                    if (row0 + 32 < N) colsel |= static_cast<uint64_t>(sb[(row0 >> 5) + 1]) << 32;
                }
                colsel >>= 4 * g;
                const uint32_t cs_lo = (uint32_t)colsel, cs_hi = (uint32_t)(colsel >> 32);
                const int lim = limit - row0, g4 = 4 * g;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int bit = kt * 16 + r;
                        const uint32_t w = bit < 32 ? cs_lo : cs_hi;
                        const bool valid = g4 < (pair ? lim_h[kt >> 1] : lim) - bit && !((w >> (bit & 31)) & 1u) &&
                                           ((halves >> (kt >> 1)) & 1u);
                        if (!valid) sacc[kt][0][r] = sacc[kt][1][r] = -INFINITY;
                    }
            }

            // online softmax in base 2 with a lazily raised reference max
            // (it moves only when a row max exceeds it by more than 8, so
            // every weight stays <= 2^8; any reference cancels in O / l)
            const float cl2 = a.c_log2e;
            float mx[2];
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                float v = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
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
                }
#pragma unroll
                for (int dt = 0; dt <= S::NDT; ++dt) {
                    o[dt][0] *= alpha[0];
                    o[dt][1] *= alpha[1];
                }
            }
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                const float neg_m = m_run[qt] == -INFINITY ? 0.0f : -m_run[qt];
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sacc[kt][qt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][qt][r], cl2, neg_m));
            }

            // weight row of this tile: 1 per token; n_j per pooled key (B, or
            // n_last for the ragged last block when this tile holds it)
            u32x4_t wrow[2];
            {
                const uint32_t w2 = approx ? blk2 : one2;
                wrow[0] = wrow[1] = u32x4_t{w2, w2, w2, w2};
                const int jlast = N - 1 - row0;
                if (approx && a.nlast != BLK && jlast >= 0 && jlast < 64 && l16 == 0) {
                    // k-index 8g+e of step u is key 32u + 4g + e or 32u + 16 + 4g + e - 4
                    const int u = jlast >> 5, rem = jlast & 31;
                    const int gl = (rem & 15) >> 2, e = (rem & 3) + (rem >= 16 ? 4 : 0);
                    if (g == gl) {
                        u16 wv[8];
#pragma unroll
                        for (int x = 0; x < 8; ++x) wv[x] = static_cast<u16>(blk2 & 0xFFFFu);
#pragma unroll
                        for (int x = 0; x < 8; ++x)
                            if (x == e) wv[x] = static_cast<u16>(pack_bf16x2(static_cast<float>(a.nlast), 0.f) & 0xFFFFu);
                        wrow[u] = u32x4_t{wv[0] | (uint32_t(wv[1]) << 16), wv[2] | (uint32_t(wv[3]) << 16),
                                          wv[4] | (uint32_t(wv[5]) << 16), wv[6] | (uint32_t(wv[7]) << 16)};
                    }
                }
            }

            // O^T += V^T P^T.  k-index 8g+e of 32-key step u is key 32u + 4g + e
            // (e < 4) or 32u + 16 + 4g + (e - 4): the keys this lane holds.
            // The transposing read gives lane (l16, g) four keys of column
            // d = 16 dt + l16 from the row addresses of lanes 16g + p + 4e.
            u32x4_t pb[2][2];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
                    pb[u][qt] = u32x4_t{pack_bf16x2(sacc[2 * u][qt][0], sacc[2 * u][qt][1]),
                                        pack_bf16x2(sacc[2 * u][qt][2], sacc[2 * u][qt][3]),
                                        pack_bf16x2(sacc[2 * u + 1][qt][0], sacc[2 * u + 1][qt][1]),
                                        pack_bf16x2(sacc[2 * u + 1][qt][2], sacc[2 * u + 1][qt][3])};
            // V^T operands in batches of VB d-tiles (batch b: 32-key step
            // u = b / NVB, d-tiles VB (b % NVB) ...); batch b+1 is read
            // before the MFMAs of batch b (ordered, as above, by the
            // compiler's interleaving strategy 1).
            constexpr int VB = S::NDT >= 4 ? 4 : S::NDT;
            constexpr int NVB = S::NDT / VB;
            bf16x8_t vfr[2][VB];
            auto vread = [&](int b, bf16x8_t (&dst)[VB]) __attribute__((always_inline)) {
                const int u = b / NVB, d0 = (b % NVB) * VB;
#pragma unroll
                for (int db = 0; db < VB; ++db) {
                    // keys 32u + 4g + (l16 >> 2) and 16 further
                    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4_t*)(Vt + v_lane + (32 * u / S::NB) * D + 16 * (d0 + db)));
                    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4_t*)(Vt + v_lane + ((32 * u + 16) / S::NB) * D + 16 * (d0 + db)));
                    dst[db] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
            };
            vread(0, vfr[0]);
#pragma unroll
            for (int b = 0; b < 2 * NVB; ++b) {
                const int u = b / NVB, d0 = (b % NVB) * VB;
                if (b == 0) __builtin_amdgcn_iglp_opt(1);
                if (b + 1 < 2 * NVB) vread(b + 1, vfr[(b + 1) & 1]);
#pragma unroll
                for (int db = 0; db < VB; ++db) {
                    o[d0 + db][0] = mfma16(vfr[b & 1][db], as_bf16x8(pb[u][0]), o[d0 + db][0]);
                    o[d0 + db][1] = mfma16(vfr[b & 1][db], as_bf16x8(pb[u][1]), o[d0 + db][1]);
                }
                if (b % NVB == NVB - 1) {
                    o[S::NDT][0] = mfma16(as_bf16x8(wrow[u]), as_bf16x8(pb[u][0]), o[S::NDT][0]);
                    o[S::NDT][1] = mfma16(as_bf16x8(wrow[u]), as_bf16x8(pb[u][1]), o[S::NDT][1]);
                }
            }
        };

        const int TS = T * S::SUB;
        if (TS > 0) {
            w_t = word_of(0, word_raw(0));
            uint32_t extra;
            if constexpr (S::KPT == 2) {
                const TileSrc src0 = source_of(w_t, 0, extra);
                tile_issue<D>(src0, K0, V0, wave_s, dma_base + extra);
            } else {
                tile_issue<D>(source_of(w_t, 0, extra), K0, V0, wave_s, dma_base);
            }
        }
        if (TS > 1) w_t1 = word_of(1, word_raw(1));
        for (int t = 0; t < TS; t += 2) {
            step(t, K0, V0, K1, V1, TS);
            if (t + 1 < TS) step(t + 1, K1, V1, K0, V0, TS);
        }

        // ---- 3. out_r = N_r / D_r --------------------------------------------
        if (myb < nqb) {
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                // row 0 of the weight tile sits in element 0 of lanes 0..15
                const float lt = __shfl(o[S::NDT][qt][0], l16);
                const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;  // 0: nothing kept (keep-or-drop)
                const int row = r0 + qt * 16 + l16;
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
        }
        if (DENSE) break;
    }
}

// ============================================================================
// launcher
// ============================================================================
namespace {

}  // namespace

int group_cost_parts(int N, int B) {
    const int NG = (N + 128 / B - 1) / (128 / B);
    return (NG + kCostGroups - 1) / kCostGroups;
}

namespace {

int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}

template <int D, int BLK, bool DENSE, bool ROUTE = false>
hipError_t sweep_t(const AttnArgs& a, hipStream_t s) {
    using S = Sweep<D, BLK>;
    auto kern = sweep_bf16_kernel<D, BLK, DENSE, ROUTE>;
    const int NC = (a.N + S::TB - 1) / S::TB;
    // selection bits of the group's query blocks, then at most NC approximate
    // and ceil(N / KPT) exact tile-list entries (at B = 32 up to 8 more: one
    // unpaired key block per selection mask)
    const size_t dyn = DENSE ? 0 : sizeof(uint32_t) * ((size_t)S::QB * ((a.N + 31) / 32) + NC +
                                                       (a.N + S::KPT - 1) / S::KPT + (S::KPT == 2 ? 8 : 0));
    int grid;
    if (DENSE) {
        const int NG = (a.N + S::QB - 1) / S::QB;
        grid = 8 * ((a.H * NG + 7) / 8);
    } else {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, S::NT, dyn) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        grid = device_cus() * per_cu;
    }
    if (!DENSE && !ROUTE && S::QB > 1 && a.gcost) {
        const int P = group_cost_parts(a.N, BLK);
        hipLaunchKernelGGL((group_cost_kernel<S::QB>), dim3(a.H * kMaxStride * P), dim3(256), 0, s, a.sel, a.N,
                           a.W, P, a.gcost);
        hipLaunchKernelGGL(group_pick_kernel, dim3(a.H), dim3(64), 0, s, a.gcost, P, a.gstride);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(S::NT), dyn, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sweep_bf16(const AttnArgs& a, int d, int B, bool dense, hipStream_t s) {
    if (a.tau_cmp && !dense) {  // routing inside the sweep
        if (!a.kept_out) return hipErrorInvalidValue;
        if (d == 64 && B == 32) return sweep_t<64, 32, false, true>(a, s);
        if (d == 128 && B == 32) return sweep_t<128, 32, false, true>(a, s);
        if (d == 64 && B == 64) return sweep_t<64, 64, false, true>(a, s);
        if (d == 64 && B == 128) return sweep_t<64, 128, false, true>(a, s);
        if (d == 128 && B == 64) return sweep_t<128, 64, false, true>(a, s);
        if (d == 128 && B == 128) return sweep_t<128, 128, false, true>(a, s);
        return hipErrorInvalidValue;
    }
    // (the dense kernel runs with B = 64 only)
    if (d == 64 && B == 32 && !dense) return sweep_t<64, 32, false>(a, s);
    if (d == 128 && B == 32 && !dense) return sweep_t<128, 32, false>(a, s);
    if (d == 64 && B == 64) return dense ? sweep_t<64, 64, true>(a, s) : sweep_t<64, 64, false>(a, s);
    if (d == 64 && B == 128) return dense ? sweep_t<64, 128, true>(a, s) : sweep_t<64, 128, false>(a, s);
    if (d == 128 && B == 64) return dense ? sweep_t<128, 64, true>(a, s) : sweep_t<128, 64, false>(a, s);
    if (d == 128 && B == 128) return dense ? sweep_t<128, 128, true>(a, s) : sweep_t<128, 128, false>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace sol
