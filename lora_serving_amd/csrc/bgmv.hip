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
constexpr int EXPAND_GROUP = 8;     // 16-byte B loads a thread keeps in flight

__device__ __forceinline__ int slice_of(const SlotGeom &g, int64_t n)
{
    int s = 0;
    while (s + 1 < g.n_slices && n >= g.slice_start[s + 1])
        ++s;
    return s;
}

// One workgroup per (token, block of EXPAND_ROWS output rows).
//   v_j = coef_j * sum_{s < n_vsplit} vsrc[s][j][t][:]   (coef_j = scale*factor, or 1)
//   delta[n] = sum_j sum_rho B[a_j][n][rho] v_j[slice(n)*R + rho]
//   y[t][n] = bf16(base[n] + delta[n]),  base = sum of n_part fp32 partials, or y itself
__global__ __launch_bounds__(256) void expand_tokens_kernel(
    const float *__restrict__ vsrc, int n_vsplit, int apply_coef, const float *__restrict__ scale,
    int64_t T, int64_t n_out, SlotGeom g, const int32_t *__restrict__ idx, int32_t K,
    const float *__restrict__ part, int32_t n_part, uint16_t *__restrict__ y)
{
    __shared__ float delta[EXPAND_ROWS];
    __shared__ float vs[MLORA_MAX_SLICES_DEV * MLORA_MAX_RANK_DEV];
    const int64_t nblk = (n_out + EXPAND_ROWS - 1) / EXPAND_ROWS;
    const int64_t t = blockIdx.x / nblk;
    const int64_t n0 = (blockIdx.x - t * nblk) * EXPAND_ROWS;
    const int nrows = (int)min((int64_t)EXPAND_ROWS, n_out - n0);
    const int R = g.R;
    const int wd = g.n_slices * R;
    const int G = R >> 3;                 // lanes per output row (a power of two <= 64)
    const int lane = threadIdx.x & 63;
    const int r4 = threadIdx.x * 4;       // first of this thread's 4 output rows
    const bool vec = ((n_out & 3) == 0) && r4 + 3 < nrows;

    bool any = false;
    for (int j = 0; j < K; ++j)
        any |= idx[t * K + j] >= 0;
    if (!any && part == nullptr)
        return;   // accumulate mode: rows with no adapter are left untouched

    // base of this thread's rows: the first EXPAND_PQ partial loads are issued now and only
    // summed at the end, so their latency overlaps the B loads
    constexpr int EXPAND_PQ = 8;
    float4 pq[EXPAND_PQ];
    const bool use_pq = part != nullptr && vec;
    if (use_pq) {
#pragma unroll
        for (int sp = 0; sp < EXPAND_PQ; ++sp)
            if (sp < n_part)
                pq[sp] = *(const float4 *)(part + ((int64_t)sp * T + t) * n_out + n0 + r4);
    }

    for (int r = threadIdx.x; r < EXPAND_ROWS; r += blockDim.x)
        delta[r] = 0.f;

    const int64_t total = (int64_t)nrows * R;          // bf16 elements of one B block
    const int64_t step = (int64_t)blockDim.x * 8;
    for (int j = 0; j < K; ++j) {
        const int a = idx[t * K + j];
        if (a < 0)
            continue;
        const uint16_t *Bb = g.B + ((int64_t)a * n_out + n0) * R;
        for (int64_t e0 = 0; e0 < total; e0 += step * EXPAND_GROUP) {
            // B loads of this group first, then (first group only) v of this slot into LDS
            u32x4 bv[EXPAND_GROUP];
#pragma unroll
            for (int u = 0; u < EXPAND_GROUP; ++u) {
                const int64_t e = e0 + u * step + (int64_t)threadIdx.x * 8;
                bv[u] = e < total ? *(const u32x4 *)(Bb + e) : u32x4{0u, 0u, 0u, 0u};
            }
            if (e0 == 0) {
                const float coef =
                    apply_coef ? (scale ? scale[t * K + j] : 1.f) * g.factor[a] : 1.f;
                for (int c = threadIdx.x; c < wd; c += blockDim.x) {
                    float sum = 0.f;
                    for (int sp = 0; sp < n_vsplit; ++sp)
                        sum += vsrc[(((int64_t)sp * K + j) * T + t) * wd + c];
                    vs[c] = coef * sum;
                }
                lds_barrier();
            }
#pragma unroll
            for (int u = 0; u < EXPAND_GROUP; ++u) {
                const int64_t e = e0 + u * step + (int64_t)threadIdx.x * 8;
                float ps = 0.f;
                int row = 0;
                if (e < total) {
                    row = (int)(e / R);
                    const int rho0 = (int)(e - (int64_t)row * R);
                    const float *vv = vs + slice_of(g, n0 + row) * R + rho0;
                    ps += bf16_lo(bv[u].x) * vv[0];
                    ps += bf16_hi(bv[u].x) * vv[1];
                    ps += bf16_lo(bv[u].y) * vv[2];
                    ps += bf16_hi(bv[u].y) * vv[3];
                    ps += bf16_lo(bv[u].z) * vv[4];
                    ps += bf16_hi(bv[u].z) * vv[5];
                    ps += bf16_lo(bv[u].w) * vv[6];
                    ps += bf16_hi(bv[u].w) * vv[7];
                }
                for (int off = 1; off < G; off <<= 1)
                    ps += __shfl_xor(ps, off, 64);
                if (e < total && (lane & (G - 1)) == 0)
                    delta[row] += ps;
            }
        }
        lds_barrier();   // delta and vs are complete for this slot
    }
    lds_barrier();

    if (r4 < nrows) {
        float base[4] = {0.f, 0.f, 0.f, 0.f};
        if (use_pq) {
#pragma unroll
            for (int sp = 0; sp < EXPAND_PQ; ++sp)
                if (sp < n_part) {
                    base[0] += pq[sp].x;
                    base[1] += pq[sp].y;
                    base[2] += pq[sp].z;
                    base[3] += pq[sp].w;
                }
            for (int sp = EXPAND_PQ; sp < n_part; ++sp) {
                const float4 q4 = *(const float4 *)(part + ((int64_t)sp * T + t) * n_out + n0 + r4);
                base[0] += q4.x;
                base[1] += q4.y;
                base[2] += q4.z;
                base[3] += q4.w;
            }
        } else if (part != nullptr) {
            for (int sp = 0; sp < n_part; ++sp) {
                const float *pp = part + ((int64_t)sp * T + t) * n_out + n0 + r4;
                for (int q = 0; q < 4 && r4 + q < nrows; ++q)
                    base[q] += pp[q];
            }
        } else {
            const uint16_t *yy = y + t * n_out + n0 + r4;
            for (int q = 0; q < 4 && r4 + q < nrows; ++q)
                base[q] = bf16_to_f32(yy[q]);
        }
        uint16_t *yo = y + t * n_out + n0 + r4;
        if (vec) {
            const uint32_t lo = pack_bf16x2(base[0] + delta[r4], base[1] + delta[r4 + 1]);
            const uint32_t hi = pack_bf16x2(base[2] + delta[r4 + 2], base[3] + delta[r4 + 3]);
            *(u32x2 *)yo = u32x2{lo, hi};
        } else {
            for (int q = 0; q < 4 && r4 + q < nrows; ++q)
                yo[q] = f32_to_bf16(base[q] + delta[r4 + q]);
        }
    }
}

hipError_t launch_expand_tokens(const float *vsrc, int n_vsplit, int apply_coef,
                                const float *scale, int64_t T, int64_t n_out, const SlotGeom &g,
                                const int32_t *idx, int32_t K, const float *part, int32_t n_part,
                                uint16_t *y, hipStream_t stream)
{
    if (T == 0 || n_out == 0)
        return hipSuccess;
    const int64_t nblk = (n_out + EXPAND_ROWS - 1) / EXPAND_ROWS;
    hipLaunchKernelGGL(expand_tokens_kernel, dim3((unsigned)(T * nblk)), dim3(256), 0, stream,
                       vsrc, n_vsplit, apply_coef, scale, T, n_out, g, idx, K, part, n_part, y);
    return hipGetLastError();
}

}  // namespace mlora
