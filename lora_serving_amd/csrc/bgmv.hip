// BGMV ("batched gather matrix-vector") shrink and expand: every (token, slot) pair fetches its
// own adapter's rows by slot index.
//
// "Multi-LoRA Serving Explained" (sevydevy.com), six-token batching script: the gather method
// picks each token's A and B by its id (-1 = base only) and multiplies; the learning book's
// chapter "04. LoRA Serving", section 6, names the two steps shrink (x A, scaled, rank-wide)
// and expand (y += v B).  The vLLM RFC on per-request composition (Proposed Change, step 4) runs
// the K slots of a token inside one kernel pass, as both kernels here do.
//
// shrink: one workgroup (4 waves) per pair.  Lanes walk n_in in 16-byte chunks (A rows are
//   read fully coalesced), keep 16 rank rows' partial dot products in registers, fold them
//   with a wave "transpose reduction" (5 shuffle rounds leave every lane with one row's sum)
//   and then across the 4 waves through LDS in a fixed order (deterministic).
// expand: one workgroup per (token, block of output rows).  Lanes walk the contiguous
//   B[a][rows][0..R) block 16 bytes at a time, so each lane holds 8 rank entries of one row;
//   the R/8 lanes of a row finish the dot product with xor shuffles over the rank dimension.
#include "bgmv_dev.h"

namespace mlora {

__global__ __launch_bounds__(256) void shrink_pairs_kernel(const uint16_t *__restrict__ x,
                                                           int64_t T, int64_t n_in, SlotGeom g,
                                                           const int32_t *__restrict__ idx,
                                                           int32_t K,
                                                           const float *__restrict__ scale,
                                                           float *__restrict__ v)
{
    __shared__ float red[64];
    shrink_one_pair(x, T, n_in, g, idx, K, scale, v, blockIdx.x, red);
}

hipError_t launch_shrink_pairs(const uint16_t *x, int64_t T, int64_t n_in, const SlotGeom &g,
                               const int32_t *idx, int32_t K, const float *scale, float *v,
                               hipStream_t stream)
{
    const int64_t P = T * K;
    if (P == 0)
        return hipSuccess;
    hipLaunchKernelGGL(shrink_pairs_kernel, dim3((unsigned)P), dim3(256), 0, stream, x, T, n_in,
                       g, idx, K, scale, v);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
constexpr int EXPAND_ROWS = 1024;   // output rows per workgroup (256 threads x 4)

__device__ __forceinline__ int slice_of(const SlotGeom &g, int64_t n)
{
    int s = 0;
    while (s + 1 < g.n_slices && n >= g.slice_start[s + 1])
        ++s;
    return s;
}

__global__ __launch_bounds__(256) void expand_tokens_kernel(const float *__restrict__ v,
                                                            int64_t T, int64_t n_out,
                                                            SlotGeom g,
                                                            const int32_t *__restrict__ idx,
                                                            int32_t K,
                                                            const float *__restrict__ part,
                                                            int32_t n_part,
                                                            uint16_t *__restrict__ y)
{
    __shared__ float delta[EXPAND_ROWS];
    const int64_t t = blockIdx.y;
    const int64_t n0 = (int64_t)blockIdx.x * EXPAND_ROWS;
    const int nrows = (int)min((int64_t)EXPAND_ROWS, n_out - n0);
    const int R = g.R;
    const int wd = g.n_slices * R;
    const int G = R >> 3;                 // lanes per output row (power of two, <= 64)
    const int lane = threadIdx.x & 63;

    bool any = false;
    for (int j = 0; j < K; ++j)
        any |= idx[t * K + j] >= 0;
    if (!any && part == nullptr)
        return;  // accumulate mode: rows with no adapter are left untouched

    for (int r = threadIdx.x; r < EXPAND_ROWS; r += blockDim.x)
        delta[r] = 0.f;
    __syncthreads();

    for (int j = 0; j < K; ++j) {
        const int a = idx[t * K + j];
        if (a < 0)
            continue;
        const uint16_t *Bb = g.B + ((int64_t)a * n_out + n0) * R;
        const float *vt = v + ((int64_t)j * T + t) * wd;
        const int64_t total = (int64_t)nrows * R;  // bf16 elements of the block
        // the block is walked in steps of 256 lanes x 8 elements; whole rows stay inside one
        // wave because R/8 divides 64
        for (int64_t e0 = 0; e0 < total; e0 += (int64_t)blockDim.x * 8) {
            const int64_t e = e0 + (int64_t)threadIdx.x * 8;
            float part_sum = 0.f;
            int row = 0;
            if (e < total) {
                row = (int)(e / R);
                const int rho0 = (int)(e - (int64_t)row * R);
                const int sg = slice_of(g, n0 + row);
                const u32x4 bv = *(const u32x4 *)(Bb + e);
                const float *vv = vt + sg * R + rho0;
                const float4 v0 = *(const float4 *)vv;
                const float4 v1 = *(const float4 *)(vv + 4);
                part_sum += bf16_lo(bv.x) * v0.x;
                part_sum += bf16_hi(bv.x) * v0.y;
                part_sum += bf16_lo(bv.y) * v0.z;
                part_sum += bf16_hi(bv.y) * v0.w;
                part_sum += bf16_lo(bv.z) * v1.x;
                part_sum += bf16_hi(bv.z) * v1.y;
                part_sum += bf16_lo(bv.w) * v1.z;
                part_sum += bf16_hi(bv.w) * v1.w;
            }
            for (int off = 1; off < G; off <<= 1)
                part_sum += __shfl_xor(part_sum, off, 64);
            if (e < total && (lane & (G - 1)) == 0)
                delta[row] += part_sum;
        }
        __syncthreads();
    }

    // y = bf16(base + delta), 4 rows per thread
    for (int r = threadIdx.x * 4; r < nrows; r += blockDim.x * 4) {
        const int64_t n = n0 + r;
        const int cnt = min(4, nrows - r);
        float base[4] = {0.f, 0.f, 0.f, 0.f};
        if (part != nullptr) {
            for (int s = 0; s < n_part; ++s) {
                const float *pp = part + ((int64_t)s * T + t) * n_out + n;
                for (int q = 0; q < cnt; ++q)
                    base[q] += pp[q];
            }
        } else {
            const uint16_t *yy = y + t * n_out + n;
            for (int q = 0; q < cnt; ++q)
                base[q] = bf16_to_f32(yy[q]);
        }
        uint16_t *yo = y + t * n_out + n;
        for (int q = 0; q < cnt; ++q)
            yo[q] = f32_to_bf16(base[q] + delta[r + q]);
    }
}

hipError_t launch_expand_tokens(const float *v, int64_t T, int64_t n_out, const SlotGeom &g,
                                const int32_t *idx, int32_t K, const float *part, int32_t n_part,
                                uint16_t *y, hipStream_t stream)
{
    if (T == 0 || n_out == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((n_out + EXPAND_ROWS - 1) / EXPAND_ROWS), (unsigned)T);
    hipLaunchKernelGGL(expand_tokens_kernel, grid, dim3(256), 0, stream, v, T, n_out, g, idx, K,
                       part, n_part, y);
    return hipGetLastError();
}

}  // namespace mlora
