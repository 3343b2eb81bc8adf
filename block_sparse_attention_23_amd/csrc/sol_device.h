// sol_device.h -- device helpers shared by the Sol-Attn kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sol {

typedef uint16_t u16;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(u16 b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ u16 f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<u16>(u >> 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// Reductions over the four lanes l, l^16, l^32, l^48 (one query row of a
// 16x16 MFMA tile) with the gfx950 lane-swap instructions: after a swap of x
// with itself the two results hold both 16-lane (or 32-lane) halves, so
// combining them gives every lane the partner's value folded in.
__device__ __forceinline__ float max4rows(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum4rows(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16) on one wavefront.
// Lane l supplies A[l%16][8*(l/16) .. +8) and B[8*(l/16) .. +8)[l%16];
// it receives D[4*(l/16) + r][l%16] in element r.
__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ float wave_max_xor16_32(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

__device__ __forceinline__ float wave_sum_xor16_32(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// ---------------------------------------------------------------------------
// Quarter qq (d/4 consecutive floats) of a pooled row, for four lanes that
// share a row: the fp32 sweep's approximate operands.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void load_kbar_quarter(const float* __restrict__ row, int qq,
                                                  float (&kv)[D / 4]) {
    const float4* p = reinterpret_cast<const float4*>(row + qq * (D / 4));
#pragma unroll
    for (int e = 0; e < D / 16; ++e) {
        float4 t = p[e];
        kv[4 * e + 0] = t.x;
        kv[4 * e + 1] = t.y;
        kv[4 * e + 2] = t.z;
        kv[4 * e + 3] = t.w;
    }
}

// The value of lane (l ^ 1), or (l ^ 2), within each group of four lanes:
// DPP quad permutations (no LDS round trip).
__device__ __forceinline__ float quad_xor1(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// Persistent-kernel work queues: eight counters, one per XCD (workgroup w
// runs on XCD w % 8).  Queue x holds, head by head, the query blocks
// [x N / 8, (x+1) N / 8).  Returns h * N + i, or -1 once all queues are empty.
__device__ __forceinline__ int claim_item(int* queues, int H, int N) {
    const int xcd = blockIdx.x & 7;
#pragma unroll 1
    for (int t = 0; t < 8; ++t) {
        const int x = (xcd + t) & 7;
        const int lo = (x * N) >> 3, hi = ((x + 1) * N) >> 3;
        const int nx = hi - lo;
        if (nx == 0) continue;
        const int kk = atomicAdd(&queues[x], 1);
        if (kk >= 0 && kk < H * nx) return (kk / nx) * N + lo + (kk % nx);
    }
    return -1;
}

// Claims from a caller-given order instead: one counter (queues[0]) walks
// order[0 .. total-1].  Returns the item, or -1 once the order is exhausted
// (or at an entry outside 0 .. total-1, which ends the claiming workgroup).
__device__ __forceinline__ int claim_ordered(int* queues, const int* order, int total) {
    const int kk = atomicAdd(&queues[0], 1);
    if (kk < 0 || kk >= total) return -1;
    const int it = order[kk];
    return (it >= 0 && it < total) ? it : -1;
}

}  // namespace sol
