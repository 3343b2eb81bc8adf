// sol_tile.h -- K/V tile machinery shared by the bf16 sweeps (gfx950):
// the LDS layout of a 64-key tile of K and V rows, and the direct-to-LDS
// buffer loads that fill it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sol_device.h"

namespace sol {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// LDS layout and direct-load split of one 64-key tile of K and V rows at
// head dimension D, for a workgroup of 256 threads.
template <int D>
struct TileLayout {
    static constexpr int NT = 256;                      // 4 waves
    static constexpr int CH = D / 8;                    // 16-byte chunks per row
    static constexpr int LPT = (64 * D * 2) / (NT * 16);  // direct loads per thread per tile
    static constexpr int NS = D / 32;                   // 32-deep steps over d
    static constexpr int NDT = D / 16;                  // 16-wide d tiles of O^T
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
template <int D>
__device__ __forceinline__ uint32_t dma_lane_base(int wave, int lane) {
    using S = TileLayout<D>;
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
template <int D, int I = 0, int IEND = TileLayout<D>::LPT>
__device__ __forceinline__ void tile_issue(const TileSrc& src, u16* Kdst, u16* Vdst, int wave_s,
                                           uint32_t lane_base) {
    if constexpr (I < IEND) {
#if defined(__HIP_DEVICE_COMPILE__)
        using S = TileLayout<D>;
        const int b = wave_s * S::LPT + I;
        const uint32_t off = lane_base + 2u * D * I;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src.k, (lds_void_t*)(Kdst + S::kbase(b)), 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src.v, (lds_void_t*)(Vdst + b * (512 + S::VPAD)), 16, off, 0, 0, 0);
#endif
        tile_issue<D, I + 1, IEND>(src, Kdst, Vdst, wave_s, lane_base);
    }
}

}  // namespace sol
