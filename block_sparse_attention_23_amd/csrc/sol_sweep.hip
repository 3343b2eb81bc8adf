// sol_sweep.hip -- the fused Sol-Attn sweep for bf16 inputs on gfx950.
//
// A workgroup (4 waves) owns 128 query rows at a time: four 32-row query
// blocks (B = 32), two 64-row blocks (B = 64) or one 128-row block
// (B = 128).  Wave w owns rows 32w .. 32w+31 as two 16-row tiles of
// v_mfma_f32_16x16x32_bf16.
//
// Per workgroup ("Sol-Attn" visual explainer, "The complete idea in one
// pass", Eq. (4), Eq. (9), Eq. (10), Eq. (11)):
//   1. the tile list: the routing kernel's selection bits of the two query
//      blocks (bit j of block i is s_ij > tau_i) are copied to LDS; a tile
//      list follows: one approximate entry per chunk of max(B, 64) pooled
//      keys that holds an unselected block of a query block, then one exact
//      entry per key block that a query block selected (the union, so a key
//      block chosen by several is loaded once; at B = 32, one 64-key tile per
//      two consecutive key blocks of the union), each tagged with the query
//      blocks that use it (at B = 32 each wave reads its own block's bits).
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
// Scheduling: persistent workgroups pull 128-row groups from eight work
// queues, one per XCD (workgroup w runs on XCD w % 8).  Queue x holds, head
// by head, the groups [x G / 8, (x+1) G / 8) of the head's G groups, so the
// workgroups of one XCD work on neighbouring rows of the same head at the
// same time and share its L2.  Every workgroup exits once all eight queues
// are drained.  Dense mode: every key block exact, no routing, one group per
// workgroup.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sol_device.h"
#include "sol_launch.h"

namespace sol {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

template <int D, int BLK>
struct Sweep {
    static constexpr int NT = 256;                      // 4 waves
    static constexpr int QB = 128 / BLK;                // query blocks per workgroup
    static constexpr int TB = BLK < 64 ? 64 : BLK;      // tokens (or pooled keys) per tile-list entry
    static constexpr int SUB = TB / 64;                 // 64-key tiles per entry
    static constexpr int KPT = BLK < 64 ? 64 / BLK : 1;  // key blocks per exact 64-key tile (2 at B = 32)
    // tile-list entry: bit 31 approximate; bits PS .. 30 the query blocks
    // that use it; bits 0 .. PS-1 the chunk or key block index.  Exact
    // entries at B = 32 instead hold two key blocks: j1 in bits 0 .. 12, j2
    // in bits 13 .. 25, bit 26 set when j2 is present.
    static constexpr int PB = QB < 2 ? 2 : QB;
    static constexpr int PS = 31 - PB;
    static constexpr int CH = D / 8;                    // 16-byte chunks per row
    static constexpr int RPK = 1024 / (2 * D);          // rows per 1 KB of LDS
    static constexpr int LPT = (64 * D * 2) / (NT * 16);  // direct loads per thread per tile
    static constexpr int NS = D / 32;                   // 32-deep steps over d
    static constexpr int NDT = D / 16;                  // 16-wide d tiles of O^T
    static constexpr int TILE = 64 * D;                 // elements of a K (or V) tile
    // LDS layout of the K (or V) rows of a tile: NB blocks of 1 KB plus
    // padding; key k is row k / NB of block k % NB.
    static constexpr int NB = 64 * 2 * D / 1024;        // blocks per tile half
    static constexpr int VPAD = 16;                      // V padding per block (elements)
    // first element of K block b: 1 KB per block plus 32 bytes per block at
    // d = 128; at d = 64 the eight blocks start 0, 32, 64, 96, 256, 288, 320,
    // 352 bytes past their 1 KB boundaries
    static constexpr __host__ __device__ int kbase(int b) {
        return 512 * b + (D >= 128 ? 16 * b : 16 * (b & 3) + 128 * (b >> 2));
    }
    static constexpr int KSLOT = kbase(NB);              // elements of a K buffer
    static constexpr int VSLOT = NB * (512 + VPAD);      // elements of a V buffer
};

constexpr uint32_t kApprox = 0x80000000u;  // tile-list entry: approximate chunk

// LDS layout of the K rows (or V rows) of a tile, chosen so that the reads
// below avoid bank conflicts and every part of a read address other than
// the lane's own offset is an instruction immediate: key k sits in row k / NB
// of 1 KB block k % NB.  Measured on gfx950 (bank-conflict counters on these
// exact patterns), the LDS behaves as 128 four-byte banks with a 16-byte read
// served 32 lanes at a time.  V blocks are padded by 32 bytes, which keeps
// the transposing V reads conflict-free at d = 64 and d = 128.  K block b
// starts kbase(b) elements in: 32 bytes of padding per block at d = 128;
// at d = 64, where a uniform padding cannot work, the offsets put the first
// banks of the eight blocks at 0, 8, 16, 24, 64, 72, 80 and 88, so the 32
// lanes of a K read (8 blocks x 2 rows x 2 chunks) cover all 128 banks.

// Direct-to-LDS loads of a tile: load i of wave w fills block b = w*LPT + i
// of the K (and of the V) buffer -- lane l writes bytes 16 l .. 16 l + 15 of
// it, i.e. row l / CH of the block, 16-byte chunk l % CH, which holds key
// (l / CH) * NB + b.  Its source offset is the lane's offset for load 0 plus
// 2 D i bytes.
template <int D, int BLK>
__device__ __forceinline__ uint32_t dma_lane_base(int wave, int lane) {
    using S = Sweep<D, BLK>;
    return (uint32_t)(((lane / S::CH) * S::NB + wave * S::LPT) * 2 * D + 16 * (lane % S::CH));
}

// Buffer resources of one 64-row tile: rows row0 .. row0+63 of a source with
// row stride D, limited to the rows before `rows` so that loads of rows past
// the end return zero (their columns are masked).
// (The buffer-resource type exists only in the device compilation.)
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t rsrc_t;
#else
typedef void* rsrc_t;
#endif
struct TileSrc {
    rsrc_t k, v;
};

// A pointer that is the same in every lane, moved to scalar registers.
__device__ __forceinline__ void* uniform_ptr(const void* p) {
    const uint64_t x = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32));
    return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}

template <int D>
__device__ __forceinline__ TileSrc tile_src(const u16* kp, const u16* vp, int row0, int rows) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int kRawBuffer = 0x00020000;  // dword 3 of a raw (untyped) buffer resource
    // With B = 128 a key block is two 64-row tiles, and the second can start
    // at or past the end of its source (an approximate chunk's upper half
    // when N <= 64 + 128 c, or an exact block holding <= 64 tokens): its
    // range is then 0 bytes and every load of it is dropped.
    const int nbytes = __builtin_amdgcn_readfirstlane(max(0, min(64, rows - row0)) * D * 2);
    return TileSrc{__builtin_amdgcn_make_buffer_rsrc(uniform_ptr(kp + (size_t)row0 * D), 0, nbytes, kRawBuffer),
                   __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(vp + (size_t)row0 * D), 0, nbytes, kRawBuffer)};
#else
    return TileSrc{};
#endif
}

// Buffer resources over rows 0 .. rows-1 of a source (B = 32 pairs: each
// lane adds its own row offset).
template <int D>
__device__ __forceinline__ TileSrc rows_src(const u16* kp, const u16* vp, int rows) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int kRawBuffer = 0x00020000;
    const int nbytes = __builtin_amdgcn_readfirstlane(rows * D * 2);
    return TileSrc{__builtin_amdgcn_make_buffer_rsrc(uniform_ptr(kp), 0, nbytes, kRawBuffer),
                   __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(vp), 0, nbytes, kRawBuffer)};
#else
    return TileSrc{};
#endif
}

// Issue this wave's LPT pairs of direct-to-LDS loads (one K, one V) of a
// tile, load I and then the rest.  The source step goes into the lane offset
// (an instruction offset would move the LDS destination as well).  wave_s is
// the wave index in an SGPR.
template <int D, int BLK, int I = 0, int IEND = Sweep<D, BLK>::LPT>
__device__ __forceinline__ void tile_issue(const TileSrc& src, u16* Kdst, u16* Vdst, int wave_s,
                                           uint32_t lane_base) {
    if constexpr (I < IEND) {
#if defined(__HIP_DEVICE_COMPILE__)
        using S = Sweep<D, BLK>;
        const int b = wave_s * S::LPT + I;
        const uint32_t off = lane_base + 2u * D * I;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src.k, (lds_void_t*)(Kdst + S::kbase(b)), 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src.v, (lds_void_t*)(Vdst + b * (512 + S::VPAD)), 16, off, 0, 0, 0);
#endif
        tile_issue<D, BLK, I + 1, IEND>(src, Kdst, Vdst, wave_s, lane_base);
    }
}

template <int D, int BLK, bool DENSE>
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
    uint32_t* tiles = dyn + S::QB * nwords;  // up to NC + ceil(N / KPT) entries
    const int myb = (wave * 32) / BLK;       // this wave's query block within the group
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t dma_base = dma_lane_base<D, BLK>(wave_s, lane);
    // when only one query block uses a tile, the other block's two waves
    // load the next tile alone: wave w covers the loads of waves 2 (w & 1)
    // and 2 (w & 1) + 1
    const uint32_t dma_base2 = dma_lane_base<D, BLK>(2 * (wave_s & 1), lane);
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

    for (;;) {
        int item;
        if (DENSE) {
            item = dense_item;
        } else {
            __syncthreads();
            if (tid == 0) misc_s[0] = claim_item(a.queues, H, NG);
            __syncthreads();
            item = __builtin_amdgcn_readfirstlane(misc_s[0]);
            if (item < 0) break;
        }
        const int h = item / NG, gi = item % NG;
        const int i0 = gi * S::QB;
        const int nqb = min(S::QB, N - i0);  // valid query blocks in this group
        const int q0 = gi * 128;
        const size_t head_off = (size_t)h * L * D;

        int T;
        if (DENSE) {
            T = N;
        } else {
            // ---- 1. the tile list ------------------------------------------
            // selection bits of the group's query blocks (written by the
            // routing kernel: bit j of block i is s_ij > tau_i)
            for (int t = tid; t < S::QB * nwords; t += S::NT) {
                const int b = t / nwords, w = t % nwords;
                selbits[t] = b < nqb ? a.sel[((size_t)h * N + i0 + b) * a.W + w] : 0u;
            }
            __syncthreads();
            if (wave == 0) {
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
                        uint32_t part = 0;
                        if (j < N)
                            for (int b = 0; b < nqb; ++b)
                                part |= ((selbits[b * nwords + (j >> 5)] >> (j & 31)) & 1u) << b;
                        const uint64_t m = __ballot(part != 0);
                        if (part) tiles[nt + __popcll(m & ((1ull << lane) - 1ull))] = (part << S::PS) | j;
                        nt += __popcll(m);
                    }
                } else {
                    // B = 32: union element r goes to entry r / 2, as j1 (r
                    // even) or j2 (r odd); within the one wave the j1 store
                    // precedes the j2 read-modify-write of the same entry
                    int nu = 0;
                    for (int j0 = 0; j0 < N; j0 += 64) {
                        const int j = j0 + lane;
                        bool any = false;
                        if (j < N)
                            for (int b = 0; b < nqb; ++b) any |= ((selbits[b * nwords + (j >> 5)] >> (j & 31)) & 1u) != 0;
                        const uint64_t m = __ballot(any);
                        const int r = nu + __popcll(m & ((1ull << lane) - 1ull));
                        if (any && !(r & 1)) tiles[nt + (r >> 1)] = (uint32_t)j;
                        if (any && (r & 1)) tiles[nt + (r >> 1)] |= ((uint32_t)j << 13) | (1u << 26);
                        nu += __popcll(m);
                    }
                    nt += (nu + 1) >> 1;
                }
                if (lane == 0) misc_s[1] = nt;
            }
            __syncthreads();
            T = __builtin_amdgcn_readfirstlane(misc_s[1]);
        }

        // Q fragments (B operand of S^T = K Q^T): rows q0 + 32w + 16qt + l16
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
        // (approx?, part, row0 of the tile in its source) of tile t
        auto decode = [&](uint32_t d, int t, bool& approx, uint32_t& part, int& row0) {
            approx = (d & kApprox) != 0;
            part = (d >> S::PS) & ((1u << S::PB) - 1u);
            row0 = (int)(d & ((1u << S::PS) - 1u)) * S::TB + (t % S::SUB) * 64;
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
            // B = 32 pairs: bit h of halves: this wave's query block selected
            // key block h of the pair; lim_h: keys of half h before L
            uint32_t halves = 3u;
            int lim_h[2] = {0, 0};
            if (S::KPT == 2 && !approx) {
                int j1, j2;
                bool has2;
                pair_of(w_t, j1, j2, has2);
                const uint32_t* sb = selbits + myb * nwords;
                halves = ((sb[j1 >> 5] >> (j1 & 31)) & 1u) | (has2 ? ((sb[j2 >> 5] >> (j2 & 31)) & 1u) << 1 : 0u);
                lim_h[0] = L - 32 * j1;
                lim_h[1] = L - 32 * j2 + 32;
            }
            // this wave's query block uses tile t
            const bool mine = S::KPT == 2 && !approx ? halves != 0u : ((part >> myb) & 1u) != 0u;
            if (t + 1 < TS) {  // tile t+1 streams into (Kn, Vn)
                uint32_t extra;
                if constexpr (S::KPT == 2) {
                    const TileSrc nsrc = source_of(w_t1, t + 1, extra);
                    tile_issue<D, BLK>(nsrc, Kn, Vn, wave_s, dma_base + extra);
                } else if (S::QB != 2 || part == 3u) {
                    tile_issue<D, BLK>(source_of(w_t1, t + 1, extra), Kn, Vn, wave_s, dma_base);
                } else if (!mine) {
                    tile_issue<D, BLK, 0, 2 * S::LPT>(source_of(w_t1, t + 1, extra), Kn, Vn, 2 * (wave_s & 1),
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
                tile_issue<D, BLK>(src0, K0, V0, wave_s, dma_base + extra);
            } else {
                tile_issue<D, BLK>(source_of(w_t, 0, extra), K0, V0, wave_s, dma_base);
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
    const int NC = (a.N + S::TB - 1) / S::TB;
    // selection bits of the group's query blocks, then at most NC approximate
    // and ceil(N / KPT) exact tile-list entries
    const size_t dyn = DENSE ? 0 : sizeof(uint32_t) * ((size_t)S::QB * ((a.N + 31) / 32) + NC +
                                                       (a.N + S::KPT - 1) / S::KPT);
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
    hipLaunchKernelGGL(kern, dim3(grid), dim3(S::NT), dyn, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sweep_bf16(const AttnArgs& a, int d, int B, bool dense, hipStream_t s) {
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
