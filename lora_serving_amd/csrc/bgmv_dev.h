// Device code of the per-pair LoRA shrink, shared by the BGMV kernels and the decode GEMM's
// fused launch (each translation unit gets its own copy; no relocatable device code).
#pragma once

#include "common.h"
#include "kernels.h"

namespace mlora {

__device__ __forceinline__ float dot8_bf16(const u32x4 a, const float xf[8])
{
    float s = 0.f;
    s += bf16_lo(a.x) * xf[0];
    s += bf16_hi(a.x) * xf[1];
    s += bf16_lo(a.y) * xf[2];
    s += bf16_hi(a.y) * xf[3];
    s += bf16_lo(a.z) * xf[4];
    s += bf16_hi(a.z) * xf[5];
    s += bf16_lo(a.w) * xf[6];
    s += bf16_hi(a.w) * xf[7];
    return s;
}

// 16 per-lane values -> every lane ends with the wave-wide sum of value number row_of(lane),
// row_of(lane) = 8*b5 + 4*b4 + 2*b3 + b2 (bits of the lane id).
__device__ __forceinline__ float transpose_reduce16(const float acc[16])
{
    const int lane = lane_id();
    float r8[8], r4[4], r2[2];
    const bool h5 = (lane >> 5) & 1, h4 = (lane >> 4) & 1, h3 = (lane >> 3) & 1,
               h2 = (lane >> 2) & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float keep = h5 ? acc[8 + i] : acc[i];
        const float send = h5 ? acc[i] : acc[8 + i];
        r8[i] = keep + __shfl_xor(send, 32, 64);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float keep = h4 ? r8[4 + i] : r8[i];
        const float send = h4 ? r8[i] : r8[4 + i];
        r4[i] = keep + __shfl_xor(send, 16, 64);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float keep = h3 ? r4[2 + i] : r4[i];
        const float send = h3 ? r4[i] : r4[2 + i];
        r2[i] = keep + __shfl_xor(send, 8, 64);
    }
    float r1;
    {
        const float keep = h2 ? r2[1] : r2[0];
        const float send = h2 ? r2[0] : r2[1];
        r1 = keep + __shfl_xor(send, 4, 64);
    }
    r1 += __shfl_xor(r1, 2, 64);
    r1 += __shfl_xor(r1, 1, 64);
    return r1;
}

// One pair's shrink by a 256-thread workgroup.  red: 64 floats of LDS.
__device__ __forceinline__ void shrink_one_pair(const uint16_t *__restrict__ x, int64_t T, int64_t n_in,
                                const SlotGeom &g, const int32_t *__restrict__ idx, int32_t K,
                                const float *__restrict__ scale, float *__restrict__ v,
                                int64_t p, float *red)
{
    const int64_t t = p / K;
    const int j = (int)(p - t * K);
    const int wd = g.n_slices * g.R;
    float *out = v + ((int64_t)j * T + t) * wd;
    const int a = idx[p];
    if (a < 0) {
        for (int c = threadIdx.x; c < wd; c += blockDim.x)
            out[c] = 0.f;
        return;
    }
    const float coef = (scale ? scale[p] : 1.f) * g.factor[a];
    const uint16_t *xt = x + t * n_in;
    const uint16_t *Aa = g.A + (int64_t)a * wd * n_in;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    for (int r0 = 0; r0 < wd; r0 += 16) {
        const int nr = min(16, wd - r0);
        float acc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[r] = 0.f;
        for (int64_t k = (int64_t)threadIdx.x * 8; k < n_in; k += (int64_t)blockDim.x * 8) {
            const u32x4 xv = *(const u32x4 *)(xt + k);
            float xf[8] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y),
                           bf16_lo(xv.z), bf16_hi(xv.z), bf16_lo(xv.w), bf16_hi(xv.w)};
            u32x4 av[16];
#pragma unroll
            for (int r = 0; r < 16; ++r)
                av[r] = r < nr ? *(const u32x4 *)(Aa + (int64_t)(r0 + r) * n_in + k)
                               : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[r] += dot8_bf16(av[r], xf);
        }
        const float s = transpose_reduce16(acc);
        const int row = ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 +
                        ((lane >> 2) & 1);
        if ((lane & 3) == 0)
            red[wave * 16 + row] = s;
        __syncthreads();
        if (threadIdx.x < 16 && (int)threadIdx.x < nr) {
            const int rr = threadIdx.x;
            const float tot = ((red[rr] + red[16 + rr]) + red[32 + rr]) + red[48 + rr];
            out[r0 + rr] = coef * tot;
        }
        __syncthreads();
    }
}

}  // namespace mlora
