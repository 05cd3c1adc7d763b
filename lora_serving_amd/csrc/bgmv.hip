// BGMV ("batched gather matrix-vector") shrink and expand: every (token, slot) pair fetches its
// own adapter's rows by slot index.
//
// Sources: "Multi-LoRA Serving Explained" (sevydevy.com), six-token batching example, gather
// variant (the slot id of a token selects the matrices it is multiplied with; -1 selects
// none); vLLM learning book, chapter "04. LoRA Serving", section 6 (the shrink to a rank-wide
// scaled intermediate and the expand that adds it back through B); "[RFC]: Per-request
// activation of multiple LoRA adapters with static scales", Proposed Change, step 4 (a token's
// K slots handled in one kernel pass, as both kernels here do).
//
// shrink: one workgroup (4 waves) per (pair, block of RB rows of the pair's n_slices * R rows),
//   RB = 16, 8, 4, 2 or 1 so that small batches still spread over many workgroups.  Lanes
//   walk n_in in 16-byte chunks (A rows read fully coalesced), two chunks of loads issued
//   before any is used, keep the RB rows' partial dot products in registers, fold them with a
//   wave "transpose reduction" (every lane ends with one row's sum) and then across the 4
//   waves through LDS in a fixed order (deterministic).
// expand: one workgroup per (token, block of output rows).  Lanes walk the contiguous
//   B[a][rows][0..R) block 16 bytes at a time, so each lane holds 8 rank entries of one row;
//   the R/8 lanes of a row finish the dot product with xor shuffles over the rank dimension.
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

// RB per-lane values -> every lane ends with the wave-wide sum of value number row_of(lane):
// log2(RB) halving rounds (xor 32, 16, ...: a lane keeps the half its lane bit selects and adds
// its partner's), then plain xor sums over the remaining lane bits.  row_of(lane) is read off
// the lane bits 5, 4, ... used by the halving rounds.
template <int RB>
__device__ __forceinline__ float transpose_reduce(float (&acc)[RB])
{
    const int lane = lane_id();
#pragma unroll
    for (int half = RB / 2, bit = 5; half >= 1; half >>= 1, --bit) {
        const bool hi = (lane >> bit) & 1;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float keep = hi ? acc[half + i] : acc[i];
            const float send = hi ? acc[i] : acc[half + i];
            acc[i] = keep + __shfl_xor(send, 1 << bit, 64);
        }
    }
    float r1 = acc[0];
#pragma unroll
    for (int bit = 5 - __builtin_ctz(RB); bit >= 0; --bit)
        r1 += __shfl_xor(r1, 1 << bit, 64);
    return r1;
}

template <int RB>
__device__ __forceinline__ int transpose_row(int lane)
{
    int row = 0;
#pragma unroll
    for (int l = 0; (1 << l) < RB; ++l)
        row = row * 2 + ((lane >> (5 - l)) & 1);
    return row;
}

// Workgroup = (pair p, rows r0 .. r0 + RB - 1 of the pair's n_slices * R rows of v).
template <int RB>
__global__ __launch_bounds__(256) void shrink_rows_kernel(const uint16_t *__restrict__ x,
                                                          int64_t T, int64_t n_in, SlotGeom g,
                                                          const int32_t *__restrict__ idx,
                                                          int32_t K,
                                                          const float *__restrict__ scale,
                                                          float *__restrict__ v)
{
    __shared__ float red[4 * RB];
    const int wd = g.n_slices * g.R;
    const int nrb = (wd + RB - 1) / RB;
    const int64_t p = blockIdx.x / nrb;
    const int r0 = (int)(blockIdx.x - p * nrb) * RB;
    const int nr = min(RB, wd - r0);
    const int64_t t = p / K;
    const int j = (int)(p - t * K);
    float *out = v + ((int64_t)j * T + t) * wd + r0;
    const uint16_t *xt = x + t * n_in;
    const int64_t step = (int64_t)blockDim.x * 8;
    // the first round's x chunks do not depend on the slot id: in flight before it is read
    u32x4 xv0[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t k = (int64_t)threadIdx.x * 8 + h * step;
        xv0[h] = k < n_in ? *(const u32x4 *)(xt + k) : u32x4{0u, 0u, 0u, 0u};
    }
    const int a = idx[p];
    // rows of this block below the adapter's rank (rounded to 8); the others are zero padding,
    // neither read nor multiplied
    const int r8 = a >= 0 ? slot_rank8(g.rank, a, g.R) : 0;
    uint32_t live = 0;
#pragma unroll
    for (int r = 0; r < RB; ++r)
        live |= (r < nr && (r0 + r) % g.R < r8 ? 1u : 0u) << r;
    if (live == 0) {
        if ((int)threadIdx.x < nr)
            out[threadIdx.x] = 0.f;
        return;
    }
    const uint16_t *Aa = g.A + ((int64_t)a * wd + r0) * n_in;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;

    float acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
        acc[r] = 0.f;
    // two 16-byte chunks per lane in flight: x and the live rows of both, then their products
    for (int64_t k0 = (int64_t)threadIdx.x * 8; k0 < n_in; k0 += 2 * step) {
        u32x4 xv[2], av[2][RB];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t k = k0 + h * step;
            const bool ok = k < n_in;
            if (k0 == (int64_t)threadIdx.x * 8)
                xv[h] = xv0[h];
            else
                xv[h] = ok ? *(const u32x4 *)(xt + k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int r = 0; r < RB; ++r)
                av[h][r] = ok && (live >> r & 1u) ? *(const u32x4 *)(Aa + (int64_t)r * n_in + k)
                                                  : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float xf[8] = {bf16_lo(xv[h].x), bf16_hi(xv[h].x), bf16_lo(xv[h].y),
                                 bf16_hi(xv[h].y), bf16_lo(xv[h].z), bf16_hi(xv[h].z),
                                 bf16_lo(xv[h].w), bf16_hi(xv[h].w)};
#pragma unroll
            for (int r = 0; r < RB; ++r)
                acc[r] += dot8_bf16(av[h][r], xf);
        }
    }
    const float s = transpose_reduce<RB>(acc);
    if ((lane & (64 / RB - 1)) == 0)
        red[wave * RB + transpose_row<RB>(lane)] = s;
    __syncthreads();
    if ((int)threadIdx.x < nr) {
        const int rr = threadIdx.x;
        const float coef = (scale ? scale[p] : 1.f) * g.factor[a];
        const float tot = ((red[rr] + red[RB + rr]) + red[2 * RB + rr]) + red[3 * RB + rr];
        out[rr] = coef * tot;
    }
}

hipError_t launch_shrink_pairs(const uint16_t *x, int64_t T, int64_t n_in, const SlotGeom &g,
                               const int32_t *idx, int32_t K, const float *scale, float *v,
                               hipStream_t stream)
{
    const int64_t P = T * K;
    if (P == 0)
        return hipSuccess;
    const int wd = g.n_slices * g.R;
    // rows per workgroup: the most (16, 8, 4, 2, 1) that still gives SHRINK_MIN_WG workgroups,
    // so small batches spread over many more workgroups than the chip has CUs
    constexpr int64_t SHRINK_MIN_WG = 2048;
    int RB = 16;
    while (RB > 1 && P * ((wd + RB - 1) / RB) < SHRINK_MIN_WG)
        RB >>= 1;
    const unsigned grid = (unsigned)(P * ((wd + RB - 1) / RB));
    switch (RB) {
    case 16:
        hipLaunchKernelGGL(shrink_rows_kernel<16>, dim3(grid), dim3(256), 0, stream, x, T, n_in,
                           g, idx, K, scale, v);
        break;
    case 8:
        hipLaunchKernelGGL(shrink_rows_kernel<8>, dim3(grid), dim3(256), 0, stream, x, T, n_in,
                           g, idx, K, scale, v);
        break;
    case 4:
        hipLaunchKernelGGL(shrink_rows_kernel<4>, dim3(grid), dim3(256), 0, stream, x, T, n_in,
                           g, idx, K, scale, v);
        break;
    case 2:
        hipLaunchKernelGGL(shrink_rows_kernel<2>, dim3(grid), dim3(256), 0, stream, x, T, n_in,
                           g, idx, K, scale, v);
        break;
    default:
        hipLaunchKernelGGL(shrink_rows_kernel<1>, dim3(grid), dim3(256), 0, stream, x, T, n_in,
                           g, idx, K, scale, v);
        break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// output rows per workgroup: 1024 (256 threads x 4), or 256 when that leaves too few
// workgroups for the chip (small batches)
constexpr int EXPAND_MIN_WG = 1024;
constexpr int EXPAND_GROUP = 8;     // 16-byte B loads a thread keeps in flight

__device__ __forceinline__ int slice_of(const SlotGeom &g, int64_t n)
{
    int s = 0;
    while (s + 1 < g.n_slices && n >= g.slice_start[s + 1])
        ++s;
    return s;
}

// One workgroup per (token, block of ER output rows).
//   v_j = coef_j * sum_{s < n_vsplit} vsrc[s][j][t][:]   (coef_j = scale*factor, or 1)
//   delta[n] = sum_j sum_rho B[a_j][n][rho] v_j[slice(n)*R + rho]
//   y[t][n] = bf16(base[n] + delta[n]),  base = sum of n_part fp32 partials, or y itself
template <int ER>
__global__ __launch_bounds__(256) void expand_tokens_kernel(
    const float *__restrict__ vsrc, int n_vsplit, int apply_coef, const float *__restrict__ scale,
    int64_t T, int64_t n_out, SlotGeom g, const int32_t *__restrict__ idx, int32_t K,
    const float *__restrict__ part, int32_t n_part, uint16_t *__restrict__ y)
{
    __shared__ float delta[ER];
    __shared__ float vs[MLORA_MAX_SLICES_DEV * MLORA_MAX_RANK_DEV];
    const int64_t nblk = (n_out + ER - 1) / ER;
    const int64_t t = blockIdx.x / nblk;
    const int64_t n0 = (blockIdx.x - t * nblk) * ER;
    const int nrows = (int)min((int64_t)ER, n_out - n0);
    const int R = g.R;
    const int wd = g.n_slices * R;
    const int lane = threadIdx.x & 63;
    const int r4 = threadIdx.x * 4;       // first of this thread's 4 output rows
    const bool vec = ((n_out & 3) == 0) && r4 + 3 < nrows;

    // base of this thread's rows, loaded first and only used at the end, so its latency
    // overlaps the slot map and the B loads: the first EXPAND_PQ partials, or y itself
    constexpr int EXPAND_PQ = 8;
    float4 pq[EXPAND_PQ];
    const bool use_pq = part != nullptr && vec;
    if (use_pq) {
#pragma unroll
        for (int sp = 0; sp < EXPAND_PQ; ++sp)
            if (sp < n_part)
                pq[sp] = *(const float4 *)(part + ((int64_t)sp * T + t) * n_out + n0 + r4);
    }
    const bool use_y = part == nullptr && vec;
    u32x2 yv = {0u, 0u};
    if (use_y)
        yv = *(const u32x2 *)(y + t * n_out + n0 + r4);

    bool any = false;
    for (int j = 0; j < K; ++j)
        any |= idx[t * K + j] >= 0;
    if (!any && part == nullptr)
        return;   // accumulate mode: rows with no adapter are left untouched

    // the first slot with an adapter stores its row sums, later ones add theirs (a row's sum
    // is always written by the same thread); with no adapter at all delta stays zero
    if (!any)
        for (int r = threadIdx.x; r < ER; r += blockDim.x)
            delta[r] = 0.f;
    bool first = true;

    const int64_t step = (int64_t)blockDim.x * 8;
    for (int j = 0; j < K; ++j) {
        const int a = idx[t * K + j];
        if (a < 0)
            continue;
        // this adapter's columns: the smallest power of two at or above its rank (rounded to
        // 8), never above R; the columns past it are zero padding and are not read.  Up to
        // R = 32 a row is at most 64 bytes, inside one cache line that is fetched whole either
        // way: all R columns are walked then, and the rank's load stays off the B loads' path
        const int r8 = R <= 32 ? R : slot_rank8(g.rank, a, R);
        int lw = 3;                                     // log2 of the columns walked per row
        while ((1 << lw) < r8)
            ++lw;
        const int RW = 1 << lw;
        const int G = RW >> 3;                          // lanes per output row
        const int total = nrows << lw;                  // elements of the block walked
        const uint16_t *Bb = g.B + ((int64_t)a * n_out + n0) * R;
        for (int e0 = 0; e0 < total; e0 += (int)step * EXPAND_GROUP) {
            // B loads of this group first, then (first group only) v of this slot into LDS
            u32x4 bv[EXPAND_GROUP];
#pragma unroll
            for (int u = 0; u < EXPAND_GROUP; ++u) {
                const int e = e0 + u * (int)step + (int)threadIdx.x * 8;
                const int row = e >> lw;
                bv[u] = e < total ? *(const u32x4 *)(Bb + (int64_t)row * R + (e & (RW - 1)))
                                  : u32x4{0u, 0u, 0u, 0u};
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
                const int e = e0 + u * (int)step + (int)threadIdx.x * 8;
                float ps = 0.f;
                int row = 0;
                if (e < total) {
                    row = e >> lw;
                    const int rho0 = e & (RW - 1);
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
                    delta[row] = first ? ps : delta[row] + ps;
            }
        }
        first = false;
        lds_barrier();   // vs is free again for the next slot
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
        } else if (use_y) {
            base[0] = bf16_lo(yv.x);
            base[1] = bf16_hi(yv.x);
            base[2] = bf16_lo(yv.y);
            base[3] = bf16_hi(yv.y);
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
    if (T * ((n_out + 1023) / 1024) >= EXPAND_MIN_WG) {
        const int64_t nblk = (n_out + 1023) / 1024;
        hipLaunchKernelGGL(expand_tokens_kernel<1024>, dim3((unsigned)(T * nblk)), dim3(256), 0,
                           stream, vsrc, n_vsplit, apply_coef, scale, T, n_out, g, idx, K, part,
                           n_part, y);
    } else {
        const int64_t nblk = (n_out + 255) / 256;
        hipLaunchKernelGGL(expand_tokens_kernel<256>, dim3((unsigned)(T * nblk)), dim3(256), 0,
                           stream, vsrc, n_vsplit, apply_coef, scale, T, n_out, g, idx, K, part,
                           n_part, y);
    }
    return hipGetLastError();
}

}  // namespace mlora
