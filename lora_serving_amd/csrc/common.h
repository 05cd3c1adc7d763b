// Device-side helpers shared by the gfx950 kernels of libmlora.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define MLORA_WAVE 64

namespace mlora {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// low / high bf16 of a packed dword
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// Mask of the lanes whose `key` (< 2^nbits) equals this lane's, using one ballot per key bit.
__device__ __forceinline__ uint64_t match_key(uint32_t key, int nbits)
{
    uint64_t m = ~0ull;
    for (int i = 0; i < nbits; ++i) {
        const bool bit = (key >> i) & 1u;
        const uint64_t b = ballot64(bit);
        m &= bit ? b : ~b;
    }
    return m;
}

// Sum over the 64 lanes of a wave (result in every lane).
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ int wave_sum_int(int v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// Exclusive prefix sum of one int per lane across the wave; *total gets the wave's sum.
__device__ __forceinline__ int wave_exclusive_scan(int v, int *total)
{
    const int lane = lane_id();
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off)
            incl += o;
    }
    *total = __shfl(incl, 63, 64);
    return incl - v;
}

// True rank of slot a, rounded up to a multiple of 8 (the 16-byte chunk of the kernels' loads;
// the slot's padding beyond the rank is zero, so the rounding adds exact zeros): R when the
// slot set has no rank table, never more than R.
__device__ __forceinline__ int slot_rank8(const int32_t *rank, int a, int R)
{
    return rank == nullptr ? R : min(R, (max(rank[a], 1) + 7) & ~7);
}

// s_barrier that waits only for this wave's LDS operations, not for its outstanding global
// loads (a __syncthreads fence waits for every outstanding memory operation); the "memory"
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace mlora
